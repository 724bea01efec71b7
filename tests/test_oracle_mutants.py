"""The oracle's pins must catch plausible mistakes.

Each case copies ``oracle/`` to a temporary folder, plants one mistake in
the copy of oracle.c (a dropped term, a wrong sign, a wrong index, a
transposed operand, a swapped coefficient), builds it, and runs a compact set
of the same independent checks used in the other oracle tests (dense LAPACK
solves, the single-mode decay of the hyperdiffusion step).  Every mutant must
fail at least one check, and the unmodified copy must pass all of them."""
import importlib.util
import os
import shutil
import sys

import numpy as np
import pytest

from dense import cyclic_dense, hines_dense, penta_dense, relerr

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTANTS = {
    "alpha_drops_a_delta_term": ("alpha[i] = c[i] - a[i] * delta[i - 2] - beta[i] * gamma[i - 1];\n        CHECK(i);\n        gamma[i] = (d[i] - beta[i] * delta[i - 1]) / alpha[i];\n        delta[i] = e[i] / alpha[i];",
                                 "alpha[i] = c[i] - beta[i] * gamma[i - 1];\n        CHECK(i);\n        gamma[i] = (d[i] - beta[i] * delta[i - 1]) / alpha[i];\n        delta[i] = e[i] / alpha[i];"),
    "gamma_wrong_sign": ("gamma[i] = (d[i] - beta[i] * delta[i - 1]) / alpha[i];\n        delta[i] = e[i] / alpha[i];",
                         "gamma[i] = (d[i] + beta[i] * delta[i - 1]) / alpha[i];\n        delta[i] = e[i] / alpha[i];"),
    "beta_wrong_index": ("beta[i] = b[i] - a[i] * gamma[i - 2];\n        alpha[i]",
                         "beta[i] = b[i] - a[i] * gamma[i - 1];\n        alpha[i]"),
    "forward_wrong_index": ("eps[i] * g[i - 2]", "eps[i] * g[i - 1]"),
    "backward_wrong_index": ("delta[i] * x[i + 2]", "delta[i] * x[i + 1]"),
    "last_row_drops_term": ("    i = n - 1;\n    beta[i] = b[i] - a[i] * gamma[i - 2];\n    alpha[i] = c[i] - a[i] * delta[i - 2] - beta[i] * gamma[i - 1];",
                            "    i = n - 1;\n    beta[i] = b[i] - a[i] * gamma[i - 2];\n    alpha[i] = c[i] - beta[i] * gamma[i - 1];"),
    "G_transposed_with_F": ("s->G0[i] = cyc_entry(n, a, b, c, d, e, m, i);",
                            "s->G0[i] = cyc_entry(n, a, b, c, d, e, i, m);"),
    "navon_rhs_sign": ("double r0 = f[m] - s0", "double r0 = f[m] + s0"),
    "schur_inverse_sign": ("s->Sinv[1] = -S[1] / det;", "s->Sinv[1] = S[1] / det;"),
    "E_used_for_E_transpose": ("ta[i] = (i >= 2) ? s->Ee[i - 2] : 0.0;", "ta[i] = (i >= 2) ? s->Ea[i] : 0.0;"),
    "F_modification_dropped": ("s->tmp[i] = f[i] - s->F0[i] * xt0 - s->F1[i] * xt1;",
                               "s->tmp[i] = f[i] - s->F0[i] * xt0;"),
    "hyperdiffusion_stencil_coefficient": ("own[2 * n + i] = 1.0 + 6.0 * sigma;", "own[2 * n + i] = 1.0 + 4.0 * sigma;"),
    "theta_sides_swapped": ("(dx * dx * dx * dx);\n    const double si = theta * sigma, se = (1.0 - theta) * sigma;",
                            "(dx * dx * dx * dx);\n    const double se = theta * sigma, si = (1.0 - theta) * sigma;"),
    "theta_stencil_neighbour_sign": ("(dx * dx * dx * dx);\n    const double si = theta * sigma, se = (1.0 - theta) * sigma;\n    const double e2 = -se, e1 = 4.0 * se,",
                                     "(dx * dx * dx * dx);\n    const double si = theta * sigma, se = (1.0 - theta) * sigma;\n    const double e2 = -se, e1 = -4.0 * se,"),
    "theta_stencil_wrong_index": ("const double xp1 = x[(i + 1) % n], xp2 = x[(i + 2) % n];",
                                  "const double xp1 = x[(i + 1) % n], xp2 = x[(i + 1) % n];"),
    "ch_phase_term_sign": ("rhs[i] = lin + r * lap;", "rhs[i] = lin - r * lap;"),
    "ch_square_for_cube": ("phi[i] = x[i] * x[i] * x[i] - x[i];", "phi[i] = x[i] * x[i] - x[i];"),
    "ch_laplacian_centre": ("const double lap = phi[im1] - 2.0 * phi[i] + phi[ip1];",
                            "const double lap = phi[im1] - 2.0 * phi[i] + phi[ip2];"),
    "ch_r_uses_dx4": ("const double r = mobility * dt / (dx * dx);",
                      "const double r = mobility * dt / (dx * dx * dx * dx);"),
    "thomas_pivot_drops_coupling": ("const double den = b[i] - cp[i - 1] * a[i];",
                                    "const double den = b[i];"),
    "thomas_rhs_wrong_index": ("y[i] = (y[i] - y[i - 1] * a[i]) / den;",
                               "y[i] = (y[i] - y[i - 1] * a[i - 1]) / den;"),
    "thomas_back_sign": ("for (int64_t i = n - 2; i >= 0; --i) y[i] = y[i] - cp[i] * y[i + 1];",
                         "for (int64_t i = n - 2; i >= 0; --i) y[i] = y[i] + cp[i] * y[i + 1];"),
    "hines_rhs_uses_parent_value": ("rhs[p[i]] -= factor * rhs[i];", "rhs[p[i]] -= factor * rhs[p[i]];"),
    "hines_forward_u_for_l": ("rhs[i] -= l[i] * rhs[p[i]];", "rhs[i] -= u[i] * rhs[p[i]];"),
    "hines_d_update_uses_u": ("d[p[i]] -= factor * l[i];", "d[p[i]] -= factor * u[i];"),
    "hines_root_division_dropped": ("    rhs[0] /= d[0];\n", "\n"),
}


def _load_copy(tmpdir, name, mutation):
    dst = os.path.join(tmpdir, name)
    shutil.copytree(ORACLE_DIR, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    src = os.path.join(dst, "oracle.c")
    text = open(src).read()
    if mutation is not None:
        old, new = mutation
        assert text.count(old) == 1, f"mutation anchor for {name} not unique/found"
        text = text.replace(old, new)
        open(src, "w").write(text)
    spec = importlib.util.spec_from_file_location(f"oracle_copy_{name}", os.path.join(dst, "__init__.py"),
                                                  submodule_search_locations=[dst])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    mod.build()
    return mod


def _checks(orc):
    """Compact pins; returns the names of the checks that fail."""
    failed = []
    rng = np.random.default_rng(0)
    # pentadiagonal, random non-symmetric dominant
    n = 9
    a, b, c, d, e = (rng.uniform(-1, 1, n) for _ in range(5))
    a[:2] = 0; b[0] = 0; d[-1] = 0; e[-2:] = 0
    c = 1 + np.abs(a) + np.abs(b) + np.abs(d) + np.abs(e) + rng.uniform(0, 1, n)
    f = rng.uniform(-1, 1, n)
    x, _ = orc.penta_solve(a, b, c, d, e, f)
    if relerr(x, np.linalg.solve(penta_dense(a, b, c, d, e), f)) > 1e-12:
        failed.append("penta_dense")
    # periodic, non-symmetric
    n = 11
    dg = [rng.uniform(-1, 1, n) for _ in range(5)]
    dg[2] = 1 + sum(np.abs(v) for k, v in enumerate(dg) if k != 2) + rng.uniform(0, 1, n)
    f = rng.uniform(-1, 1, n)
    x, _ = orc.penta_cyclic_solve(*dg, f)
    if relerr(x, np.linalg.solve(cyclic_dense(*dg), f)) > 1e-12:
        failed.append("cyclic_dense")
    # hyperdiffusion single-mode decay
    N, dt = 64, 1e-6
    sigma = dt * N ** 4
    xs = np.arange(N) / N
    C0 = np.cos(2 * np.pi * 3 * xs)
    C = orc.hyperdiffusion(C0, dt, 1.0 / N, 2)[0]
    g = 1 / (1 + sigma * (2 - 2 * np.cos(2 * np.pi * 3 / N)) ** 2)
    if np.max(np.abs(C - g ** 2 * C0)) > 1e-10:
        failed.append("mode_decay")
    # theta scheme (theta != 1/2, so that the two sides differ): one step of a
    # random state vs dense solves
    n, dt = 9, 0.02
    (e2, e1, e0), dgt = orc.hyperdiffusion_theta_operators(n, dt, 1.0 / n, 0.3)
    Bt = np.zeros((n, n))
    for i in range(n):
        for off, v in ((-2, e2), (-1, e1), (0, e0), (1, e1), (2, e2)):
            Bt[i, (i + off) % n] += v
    C0 = rng.uniform(-1, 1, n)
    got = orc.hyperdiffusion_theta(C0, dt, 1.0 / n, 0.3, 1)[0]
    if relerr(got, np.linalg.solve(cyclic_dense(*dgt), Bt @ C0)) > 1e-12:
        failed.append("theta_dense")
    # Cahn-Hilliard: one step vs dense solves with the phase-separation term
    n, dt, dx, gm, mob = 9, 2e-3, 1.0 / 9, 0.05, 1.3
    (e2, e1, e0), r, dgc = orc.cahn_hilliard_operators(n, dt, dx, gm, mob, 0.5)
    Bc = np.zeros((n, n)); L2 = np.zeros((n, n))
    for i in range(n):
        for off, v in ((-2, e2), (-1, e1), (0, e0), (1, e1), (2, e2)):
            Bc[i, (i + off) % n] += v
        for off, v in ((-1, 1.0), (0, -2.0), (1, 1.0)):
            L2[i, (i + off) % n] += v
    C0 = rng.uniform(-1, 1, n)
    got = orc.cahn_hilliard(C0, dt, dx, gm, mob, 0.5, 1)[0]
    ref = np.linalg.solve(cyclic_dense(*dgc), Bc @ C0 + r * (L2 @ (C0 ** 3 - C0)))
    if relerr(got, ref) > 1e-12:
        failed.append("ch_dense")
    # Thomas, random dominant tridiagonal
    n = 10
    ta, tc = rng.uniform(-1, 1, (2, n))
    ta[0] = tc[-1] = 0
    tbd = 1 + np.abs(ta) + np.abs(tc) + rng.uniform(0, 1, n)
    ty = rng.uniform(-1, 1, n)
    u, _ = orc.thomas_solve(ta, tbd, tc, ty)
    A = np.diag(tbd) + np.diag(ta[1:], -1) + np.diag(tc[:-1], 1)
    if relerr(u[0], np.linalg.solve(A, ty)) > 1e-12:
        failed.append("thomas_dense")
    # Hines, random tree, u != l
    from workloads import random_tree
    p = random_tree(30, rng, window=4)
    u = rng.uniform(-1, 0, 30); l = rng.uniform(-1, 0, 30); u[0] = l[0] = 0
    dd = 1 + np.abs(l) + rng.uniform(0, 1, 30)
    for i in range(1, 30):
        dd[p[i]] += abs(u[i])
    f = rng.uniform(-1, 1, 30)
    V, _ = orc.hines_solve(p, u, l, dd, f)
    if relerr(V, np.linalg.solve(hines_dense(p, u, l, dd), f)) > 1e-12:
        failed.append("hines_dense")
    return failed


def test_unmodified_copy_passes(tmp_path):
    orc = _load_copy(str(tmp_path), "clean", None)
    assert _checks(orc) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    orc = _load_copy(str(tmp_path), name, MUTANTS[name])
    assert _checks(orc), f"planted mistake {name} was not caught by any pin"
