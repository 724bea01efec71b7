"""Pins for the oracle's Thomas algorithm (Hines page, section 4.1: forward
elimination of the lower diagonal, backward substitution; the method of
cuThomasBatch).

Independent checks: scipy's banded LAPACK solver (gbsv-type, partial
pivoting) on random dominant systems of many sizes, exact rational solutions
of small integer systems (tests/golden/exact_tri.json, written by the
referee's exact Gaussian elimination), the Hines solver on a chain tree
(elimination in the opposite order: leaves to root is last row to first),
closed forms (the second-difference matrix and a diagonal matrix), info on
a zero pivot, and residuals at the page's largest sizes."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads as W
from dense import relerr

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _banded(a, b, c):
    n = len(b)
    ab = np.zeros((3, n))
    ab[0, 1:] = c[:-1]
    ab[1] = b
    ab[2, :-1] = a[1:]
    return ab


@pytest.mark.parametrize("n", [1, 2, 3, 5, 16, 64, 511, 2048])
def test_matches_lapack_banded(n):
    tb = W.tri_dominant(n, 6, rng=np.random.default_rng(n))
    u, info = oracle.thomas_solve(*(W.to_flat(v) for v in (tb.a, tb.b, tb.c, tb.y)))
    assert np.all(info == 0)
    for s in range(6):
        xr = scipy.linalg.solve_banded((1, 1), _banded(tb.a[:, s], tb.b[:, s], tb.c[:, s]), tb.y[:, s])
        assert relerr(u[s], xr) < 1e-14


def test_random_sign_diagonal_dense():
    """Dominant but with negative diagonal entries: dense LAPACK."""
    rng = np.random.default_rng(3)
    n = 40
    a, c = rng.uniform(-1, 1, (2, n))
    a[0] = c[-1] = 0
    b = (1 + np.abs(a) + np.abs(c)) * np.where(rng.random(n) < 0.5, -1, 1)
    y = rng.uniform(-1, 1, n)
    A = np.diag(b) + np.diag(a[1:], -1) + np.diag(c[:-1], 1)
    u, _ = oracle.thomas_solve(a, b, c, y)
    assert relerr(u[0], np.linalg.solve(A, y)) < 1e-14


def test_exact_integer_systems_golden():
    with open(os.path.join(GOLDEN, "exact_tri.json")) as fh:
        cases = json.load(fh)["cases"]
    assert len(cases) >= 15
    for cs in cases:
        u, info = oracle.thomas_solve(*(np.array(cs[k], float) for k in ("a", "b", "c", "f")))
        xe = np.array([float(Fraction(v)) for v in cs["x"]])
        assert info[0] == 0
        assert np.max(np.abs(u[0] - xe)) <= 1e-14 * max(1.0, np.max(np.abs(xe)))


def test_outside_entries_ignored():
    rng = np.random.default_rng(4)
    tb = W.tri_dominant(9, 3, rng=rng)
    a, b, c, y = (W.to_flat(v) for v in (tb.a, tb.b, tb.c, tb.y))
    u0, _ = oracle.thomas_solve(a, b, c, y)
    a2, c2 = a.copy(), c.copy()
    a2[:, 0] = 123.0
    c2[:, -1] = -77.0
    u1, _ = oracle.thomas_solve(a2, b, c2, y)
    np.testing.assert_array_equal(u0, u1)


def test_chain_tree_hines_agrees():
    """A chain tree p_i = i - 1 is tridiagonal with u_i = c_{i-1}, l_i = a_i;
    the Hines solver eliminates from the last row upwards."""
    n = 300
    tb = W.tri_dominant(n, 4, rng=np.random.default_rng(5))
    a, b, c, y = (W.to_flat(v) for v in (tb.a, tb.b, tb.c, tb.y))
    u, _ = oracle.thomas_solve(a, b, c, y)
    p = np.arange(-1, n - 1, dtype=np.int32)
    hu = np.zeros_like(a)
    hu[:, 1:] = c[:, :-1]
    V, _ = oracle.hines_solve(p, hu, a, b, y)
    assert relerr(u, V) < 1e-14


def test_second_difference_closed_form():
    """-x'' = 1 on a uniform grid with zero boundary values: the discrete
    solution of tridiag(-1, 2, -1) u = h^2 is the parabola u_i = h^2 (i+1)(n-i)/2,
    exact (no truncation error for a quadratic)."""
    n = 99
    h = 1.0 / (n + 1)
    a = -np.ones(n); a[0] = 0
    c = -np.ones(n); c[-1] = 0
    b = 2 * np.ones(n)
    u, _ = oracle.thomas_solve(a, b, c, h * h * np.ones(n))
    i = np.arange(n)
    assert np.max(np.abs(u[0] - h * h * (i + 1) * (n - i) / 2)) < 1e-14


def test_diagonal_matrix():
    rng = np.random.default_rng(6)
    b = rng.uniform(1, 2, 20)
    y = rng.uniform(-1, 1, 20)
    u, _ = oracle.thomas_solve(np.zeros(20), b, np.zeros(20), y)
    np.testing.assert_allclose(u[0], y / b, rtol=1e-16, atol=0)


def test_info_reports_first_bad_pivot():
    # b_0 = 0 -> info 1; a pivot b_2 - c'_1 a_2 = 0 -> info 3
    a = np.array([0.0, 1.0, 1.0, 1.0]); b = np.array([0.0, 2.0, 2.0, 2.0]); c = np.ones(4)
    _, info = oracle.thomas_solve(a, b, c, np.ones(4))
    assert info[0] == 1
    b = np.array([1.0, 2.0, 1.0, 2.0])
    # c'_0 = 1, den_1 = 2 - 1 = 1, c'_1 = 1, den_2 = 1 - 1 = 0
    _, info = oracle.thomas_solve(a, b, c, np.ones(4))
    assert info[0] == 3


@pytest.mark.parametrize("n,batch", [(512, 64), (8192, 8)])
def test_residual_at_page_sizes(n, batch):
    tb = W.tri_dominant(n, batch, rng=np.random.default_rng(n + 1))
    a, b, c, y = (W.to_flat(v) for v in (tb.a, tb.b, tb.c, tb.y))
    u, info = oracle.thomas_solve(a, b, c, y)
    assert np.all(info == 0)
    r = b * u - y
    r[:, 1:] += a[:, 1:] * u[:, :-1]
    r[:, :-1] += c[:, :-1] * u[:, 1:]
    scale = (np.abs(a) + np.abs(b) + np.abs(c)).max(axis=1) * np.abs(u).max(axis=1)
    assert np.max(np.abs(r).max(axis=1) / scale) < 4e-16
