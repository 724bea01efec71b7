"""Pins for the oracle's periodic pentadiagonal solve (cuPentBatch page,
hyperdiffusion section: the periodic matrix and Navon's reduction, eqs.
(10)-(12)) and the implicit hyperdiffusion step built on it.

Independent checks: dense LAPACK solves of the periodic matrix, exact
rational elimination, the circulant closed form (a discrete Fourier solve
with eigenvalues lambda_k = c + 2 b cos(theta_k) + 2 a cos(2 theta_k) of the
same fp64 entries, evaluated in extended precision), the exact per-step decay
of a single Fourier mode, mean conservation, the parabolic property (the norm
never grows), the definitions of the stored reduction quantities, and the
page's own validation (harmonic solution, error ~ N^-2)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from dense import cyclic_dense, relerr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dominant_cyclic(n, rng):
    a, b, d, e = (rng.uniform(-1, 1, n) for _ in range(4))
    c = 1 + np.abs(a) + np.abs(b) + np.abs(d) + np.abs(e) + rng.uniform(0, 1, n)
    return a, b, c, d, e


@pytest.mark.parametrize("n", [6, 7, 8, 9, 12, 16, 33])
def test_matches_dense_lapack(n):
    rng = np.random.default_rng(200 + n)
    for _ in range(4):
        dg = _dominant_cyclic(n, rng)
        f = rng.uniform(-1, 1, (3, n))
        x, info = oracle.penta_cyclic_solve(*(np.tile(v, (3, 1)) for v in dg), f)
        assert np.all(info == 0)
        xr = np.linalg.solve(cyclic_dense(*dg), f.T).T
        assert relerr(x, xr) < 1e-13


def test_nonsymmetric_random_sign(n=10):
    """Non-dominant, non-symmetric periodic matrix (E^T differs from E)."""
    rng = np.random.default_rng(5)
    for _ in range(10):
        a, b, d, e = (rng.uniform(-1, 1, n) for _ in range(4))
        c = rng.choice([-1.0, 1.0], n) * rng.uniform(2.5, 4.0, n)
        A = cyclic_dense(a, b, c, d, e)
        f = rng.uniform(-1, 1, n)
        x, info = oracle.penta_cyclic_solve(a, b, c, d, e, f)
        if info[0] != 0 or np.linalg.cond(A) > 1e5:
            continue
        assert relerr(x, np.linalg.solve(A, f)) < 1e-12


def test_exact_integer_systems_golden():
    with open(os.path.join(GOLDEN, "exact_cyclic.json")) as fh:
        cases = json.load(fh)["cases"]
    assert len(cases) >= 10
    for cs in cases:
        x, info = oracle.penta_cyclic_solve(*(np.array(cs[k], float) for k in "abcdef"))
        xe = np.array([float(Fraction(v)) for v in cs["x"]])
        assert info[0] == 0
        assert np.max(np.abs(x[0] - xe)) <= 1e-13 * max(1.0, np.max(np.abs(xe)))


def test_reduction_quantities_match_their_definitions():
    """The stored rows of G E^{-1} satisfy W E = G, and the stored 2x2 block is
    the inverse of H - G E^{-1} F (blocks of the periodic matrix)."""
    rng = np.random.default_rng(9)
    n = 14
    dg = _dominant_cyclic(n, rng)
    Wr, Sinv, info = oracle.penta_cyclic_setup(*dg)
    assert info == 0
    A = cyclic_dense(*dg)
    m = n - 2
    E, F, G, H = A[:m, :m], A[:m, m:], A[m:, :m], A[m:, m:]
    np.testing.assert_allclose(Wr @ E, G, atol=1e-13)
    S = H - G @ np.linalg.solve(E, F)
    np.testing.assert_allclose(Sinv @ S, np.eye(2), atol=1e-13)


def _circulant_solve(f, a, b, c):
    """Exact circulant solve for constant symmetric diagonals (a=e, b=d)."""
    n = f.shape[-1]
    th = (2 * np.pi * np.arange(n) / n).astype(np.longdouble)
    L = np.longdouble
    lam = (L(c) + 2 * L(b) * np.cos(th) + 2 * L(a) * np.cos(2 * th)).astype(float)
    return np.real(np.fft.ifft(np.fft.fft(f, axis=-1) / lam, axis=-1))


@pytest.mark.parametrize("n,tol", [(256, 2e-12), (1024, 3e-10)])
def test_circulant_closed_form(n, tol):
    """Workload step matrices: sigma = 1e-6 * n^4 (kappa ~ 7e4 and ~ 1.8e7)."""
    a, b, c, d, e = oracle.hyperdiffusion_diagonals(n, 1e-6, 1.0 / n)
    f = np.random.default_rng(1).uniform(-1, 1, (16, n))
    x, info = oracle.penta_cyclic_solve(a, b, c, d, e, f)
    assert np.all(info == 0)
    assert relerr(x, _circulant_solve(f, a[0], b[0], c[0])) < tol


def _decay(n, dt, k):
    """Per-step factor of mode k: 1 / lambda_k with lambda_k the eigenvalue of
    the fp64 matrix.  In exact arithmetic lambda_k = 1 + sigma (2 - 2 cos
    theta)^2 (the stencil [1,-4,6,-4,1] has symbol (2 - 2 cos theta)^2); it is
    evaluated from the stored fp64 entries in extended precision, because
    rounding 1 + 6 sigma alone moves lambda_k by ~1e-12 relative."""
    a, b, c, d, e = oracle.hyperdiffusion_diagonals(n, dt, 1.0 / n)
    L = np.longdouble
    th = (2 * np.pi * np.asarray(k) / n).astype(L)
    lam = L(c[0]) + 2 * L(b[0]) * np.cos(th) + 2 * L(a[0]) * np.cos(2 * th)
    sigma = dt * n ** 4
    exact = 1 + sigma * (2 - 2 * np.cos(th.astype(float))) ** 2
    assert np.all(np.abs(lam.astype(float) / exact - 1) < 1e-10)
    return (1 / lam).astype(float)


def test_single_mode_decay_exact():
    """cos(2 pi k x_i) is an eigenvector of I + sigma D4, so each implicit
    step divides it by exactly its eigenvalue."""
    n, dt, nsteps = 256, 1e-6, 10
    dx = 1.0 / n
    x = np.arange(n) / n
    ks = np.array([1, 2, 4, 8, 16])
    C0 = np.cos(2 * np.pi * ks[:, None] * x[None, :])
    C = oracle.hyperdiffusion(C0, dt, dx, nsteps)
    g = _decay(n, dt, ks)
    np.testing.assert_allclose(C, (g ** nsteps)[:, None] * C0, rtol=0, atol=1e-11)


def test_workload0_modes_closed_form():
    ic = W.hyperdiffusion_modes(256, 64)
    n, dt = 256, 1e-6
    dx = 1.0 / n
    C = oracle.hyperdiffusion(W.to_flat(ic.C0), dt, dx, 10)
    x = np.arange(n) / n
    g = _decay(n, dt, ic.k)   # (batch, modes)
    ref = np.sum((ic.amp * g ** 10)[:, None, :] *
                 np.cos(2 * np.pi * x[None, :, None] * ic.k[:, None, :] + ic.phase[:, None, :]),
                 axis=2)
    np.testing.assert_allclose(C, ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("n,rtol", [(256, 1e-11), (1024, 3e-10)])
def test_mean_conserved_and_norm_non_increasing(n, rtol):
    """Rows of I + sigma D4 sum to one and the matrix is symmetric, so each
    step keeps sum(C).  With the fp64 entries the row sum is
    lambda_0 = a + b + c + d + e (1 + 4.7e-10 at n = 1024, from rounding
    1 + 6 sigma), and the exact statement is sum(C^{k+1}) = sum(C^k) / lambda_0.
    The tolerance is the solver's rounding at kappa ~ 7e4 and ~ 1.8e7."""
    dt, dx = 1e-6, 1.0 / n
    C = np.random.default_rng(4).uniform(-1, 1, (8, n)) + 0.3
    m0 = C.sum(axis=1)
    a, b, c, d, e = oracle.hyperdiffusion_diagonals(n, dt, dx)
    L = np.longdouble
    lam0 = float(L(a[0]) + L(b[0]) + L(c[0]) + L(d[0]) + L(e[0]))
    assert abs(lam0 - 1) < 1e-9
    norms = [np.linalg.norm(C, axis=1)]
    for _ in range(5):
        C = oracle.hyperdiffusion(C, dt, dx, 1)
        norms.append(np.linalg.norm(C, axis=1))
    np.testing.assert_allclose(C.sum(axis=1), m0 / lam0 ** 5, rtol=rtol, atol=0)
    for k in range(5):
        assert np.all(norms[k + 1] <= norms[k] * (1 + 1e-14))


def test_steps_compose_bitwise():
    """k + m steps equal k steps then m steps (same operations)."""
    n = 64
    C0 = np.random.default_rng(2).uniform(-1, 1, (3, n))
    a = oracle.hyperdiffusion(C0, 1e-6, 1.0 / n, 7)
    b = oracle.hyperdiffusion(oracle.hyperdiffusion(C0, 1e-6, 1.0 / n, 3), 1e-6, 1.0 / n, 4)
    np.testing.assert_array_equal(a, b)


def test_explicit_diagonals_equal_default():
    n, dt, dx = 48, 1e-6, 1.0 / 48
    C0 = np.random.default_rng(3).uniform(-1, 1, (2, n))
    dg = oracle.hyperdiffusion_diagonals(n, dt, dx)
    np.testing.assert_array_equal(oracle.hyperdiffusion(C0, dt, dx, 3),
                                  oracle.hyperdiffusion(C0, dt, dx, 3, diagonals=dg))


def test_page_validation_harmonic_converges_second_order():
    """The page's validation: C(x,0) = A cos(k x + phi), exact decay
    exp(-k^4 t); the L2 error at T shrinks like N^-2.  The implicit step's
    own O(dt) error is made negligible with a small dt."""
    with open(os.path.join(GOLDEN, "hyperdiffusion_harmonic.json")) as fh:
        g = json.load(fh)
    k = 2 * math.pi * g["mode"] / g["L"]
    lam = k ** 4
    nsteps = 20000
    dt = g["T"] / nsteps
    errs = []
    Ns = (16, 32, 64)
    for N in Ns:
        dx = g["L"] / N
        x = np.arange(N) * dx
        C0 = g["A"] * np.cos(k * x + g["phi"])
        C = oracle.hyperdiffusion(C0, dt, dx, nsteps)[0]
        exact = g["A"] * np.cos(k * x + g["phi"]) * math.exp(-lam * g["T"])
        errs.append(math.sqrt(np.sum((C - exact) ** 2) * dx))
    orders = [math.log(errs[i] / errs[i + 1], 2) for i in range(len(Ns) - 1)]
    for p in orders:
        assert abs(p - g["expected_order"]) < 0.15, (errs, orders)
