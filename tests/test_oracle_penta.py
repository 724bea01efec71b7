"""Pins for the oracle's pentadiagonal solver (cuPentBatch page, section
"Pentadiagonal solver": factorisation steps 1-14, forward steps for g,
back-substitution steps for x).  Each check compares against something the
oracle does not compute itself: dense LAPACK solves, exact rational
elimination, the LR product re-assembled entry by entry, the tridiagonal
special case (a = e = 0) against scipy's banded solver, and residuals at the
full workload size."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads as W
from dense import penta_dense, relerr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_system(n, rng, kind):
    dg = [rng.uniform(-1, 1, n) for _ in range(5)]
    a, b, c, d, e = dg
    if kind == "dominant":
        c = 1 + np.abs(a) + np.abs(b) + np.abs(d) + np.abs(e) + rng.uniform(0, 1, n)
    elif kind == "spd":
        # symmetric: a_i = e_{i-2}, b_i = d_{i-1}; dominant diagonal -> SPD
        e = rng.uniform(-1, 1, n); d = rng.uniform(-1, 1, n)
        a = np.r_[0, 0, e[:-2]]; b = np.r_[0, d[:-1]]
        c = 1 + 2 * (np.abs(d) + np.abs(e)) + rng.uniform(0, 1, n)
    else:  # random signs, diagonal moved away from zero but not dominant
        c = np.sign(rng.uniform(-1, 1, n)) * rng.uniform(1.5, 3.0, n)
    a = a.copy(); b = b.copy(); d = d.copy(); e = e.copy()
    a[:2] = 0; b[0] = 0; d[-1] = 0; e[-2:] = 0
    return a, b, c, d, e


@pytest.mark.parametrize("kind", ["dominant", "spd", "random"])
@pytest.mark.parametrize("n", [4, 5, 6, 7, 8, 11, 16])
def test_matches_dense_lapack(n, kind):
    rng = np.random.default_rng(100 + n)
    for _ in range(4):
        a, b, c, d, e = _random_system(n, rng, kind)
        A = penta_dense(a, b, c, d, e)
        if np.linalg.cond(A) > 1e6:
            continue
        f = rng.uniform(-1, 1, (3, n))
        x, info = oracle.penta_solve(*(np.tile(v, (3, 1)) for v in (a, b, c, d, e)), f)
        assert np.all(info == 0)
        xr = np.linalg.solve(A, f.T).T
        assert relerr(x, xr) < 1e-13


def test_factors_reassemble_the_matrix():
    """L R with L = [eps=a on -2, beta on -1, alpha on 0] and
    R = [1 on 0, gamma on +1, delta on +2] must give back A."""
    rng = np.random.default_rng(7)
    for n in (4, 5, 9, 20):
        a, b, c, d, e = _random_system(n, rng, "dominant")
        al, be, ga, de, info = oracle.penta_factor(a, b, c, d, e)
        assert info == 0
        L = np.diag(al) + np.diag(be[1:], -1) + np.diag(a[2:], -2)
        R = np.eye(n) + np.diag(ga[:-1], 1) + np.diag(de[:-2], 2)
        np.testing.assert_allclose(L @ R, penta_dense(a, b, c, d, e), rtol=0, atol=1e-14)


def test_exact_integer_systems_golden():
    with open(os.path.join(GOLDEN, "exact_penta.json")) as fh:
        cases = json.load(fh)["cases"]
    assert len(cases) >= 10
    for cs in cases:
        x, info = oracle.penta_solve(*(np.array(cs[k], float) for k in "abcdef"))
        xe = np.array([float(Fraction(v)) for v in cs["x"]])
        assert info[0] == 0
        assert np.max(np.abs(x[0] - xe)) <= 1e-13 * max(1.0, np.max(np.abs(xe)))


def test_tridiagonal_special_case_matches_solve_banded():
    """a = e = 0 reduces the pentadiagonal elimination to Thomas' algorithm."""
    rng = np.random.default_rng(11)
    n = 300
    b = rng.uniform(-1, 1, n); d = rng.uniform(-1, 1, n)
    b[0] = 0; d[-1] = 0
    c = 1 + np.abs(b) + np.abs(d) + rng.uniform(0, 1, n)
    z = np.zeros(n)
    f = rng.uniform(-1, 1, n)
    x, info = oracle.penta_solve(z, b, c, d, z, f)
    ab = np.zeros((3, n)); ab[0, 1:] = d[:-1]; ab[1] = c; ab[2, :-1] = b[1:]
    xr = scipy.linalg.solve_banded((1, 1), ab, f)
    assert relerr(x, xr) < 1e-14


def test_shared_coefficients_equal_per_system():
    """Factor once and solve many (shared diagonals) == factor per system."""
    rng = np.random.default_rng(12)
    n, batch = 37, 9
    a, b, c, d, e = _random_system(n, rng, "dominant")
    f = rng.uniform(-1, 1, (batch, n))
    xs, _ = oracle.penta_solve(a, b, c, d, e, f)
    xp, _ = oracle.penta_solve(*(np.tile(v, (batch, 1)) for v in (a, b, c, d, e)), f)
    np.testing.assert_array_equal(xs, xp)


def test_zero_pivot_reported():
    n = 8
    a, b, c, d, e = (np.zeros(n) for _ in range(5))
    c[:] = 2.0
    c0 = c.copy(); c0[0] = 0.0
    _, info = oracle.penta_solve(a, b, c0, d, e, np.ones((1, n)))
    assert info[0] == 1
    # second pivot alpha_1 = c_1 - b_1 gamma_0 = 0
    d2 = d.copy(); d2[0] = 2.0
    b2 = b.copy(); b2[1] = 2.0
    _, info = oracle.penta_solve(a, b2, c, d2, e, np.ones((1, n)))
    assert info[0] == 2


@pytest.mark.slow
def test_residual_full_workload_sample():
    """Workload 2 (n=512): relative residual of sampled systems at full size."""
    pb = W.penta_dominant(512, 256, rng=np.random.default_rng(3))
    fl = [W.to_flat(v) for v in (*pb.diagonals, pb.f)]
    x, info = oracle.penta_solve(*fl)
    assert np.all(info == 0)
    for s in range(0, 256, 17):
        A = penta_dense(*(v[s] for v in fl[:5]))
        r = A @ x[s] - fl[5][s]
        assert np.max(np.abs(r)) / (np.max(np.abs(A).sum(1)) * np.max(np.abs(x[s]))) < 1e-15
