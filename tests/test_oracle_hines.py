"""Pins for the oracle's Hines solver (Hines page, section 2, Algorithm 1).

Independent checks: dense LAPACK solves of the Hines matrix on every tree
shape up to 6 compartments (all parent vectors with p_i < i), exact rational
elimination, a chain tree against scipy's tridiagonal banded solver (the
Thomas case, Hines page section 4.1), the symmetric case against a Cholesky
solve, invariance under renumbering the tree, multi-morphology batches equal
to neurons solved one by one, and residuals at full workload sizes."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads as W
from dense import hines_dense, relerr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _values(p, rng, batch=1):
    n = len(p)
    u = rng.uniform(-1, 0, (batch, n)); l = rng.uniform(-1, 0, (batch, n))
    u[:, 0] = 0; l[:, 0] = 0
    d = 1 + np.abs(l) + rng.uniform(0, 1, (batch, n))
    for i in range(1, n):
        d[:, p[i]] += np.abs(u[:, i])
    f = rng.uniform(-1, 1, (batch, n))
    return u, l, d, f


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_every_tree_shape_matches_dense(n):
    rng = np.random.default_rng(300 + n)
    ranges = [range(i) for i in range(1, n)]
    count = 0
    for tail in itertools.product(*ranges):
        p = np.array((-1,) + tail, dtype=np.int32)
        u, l, d, f = _values(p, rng)
        # also random signs on the off-diagonals
        u *= rng.choice([-1, 1], u.shape); l *= rng.choice([-1, 1], l.shape)
        V, info = oracle.hines_solve(p, u, l, d, f)
        assert info[0] == 0
        xr = np.linalg.solve(hines_dense(p, u[0], l[0], d[0]), f[0])
        assert relerr(V, xr) < 1e-14
        count += 1
    assert count == max(1, int(np.prod([len(r) for r in ranges])))


def test_exact_integer_trees_golden():
    with open(os.path.join(GOLDEN, "exact_hines.json")) as fh:
        cases = json.load(fh)["cases"]
    assert len(cases) >= 10
    for cs in cases:
        p = np.array(cs["parent"], dtype=np.int32)
        V, info = oracle.hines_solve(p, *(np.array(cs[k], float) for k in ("u", "l", "d", "f")))
        xe = np.array([float(Fraction(v)) for v in cs["x"]])
        assert info[0] == 0
        assert np.max(np.abs(V[0] - xe)) <= 1e-14 * max(1.0, np.max(np.abs(xe)))


def test_chain_tree_is_thomas():
    rng = np.random.default_rng(8)
    n = 400
    p = np.arange(-1, n - 1, dtype=np.int32)
    u, l, d, f = _values(p, rng, 4)
    V, info = oracle.hines_solve(p, u, l, d, f)
    for s in range(4):
        ab = np.zeros((3, n))
        ab[0, 1:] = u[s, 1:]       # A[i-1][i] = u_i (superdiagonal)
        ab[1] = d[s]
        ab[2, :-1] = l[s, 1:]      # A[i][i-1] = l_i (subdiagonal)
        xr = scipy.linalg.solve_banded((1, 1), ab, f[s])
        assert relerr(V[s], xr) < 1e-14


def test_symmetric_case_cholesky():
    rng = np.random.default_rng(10)
    p = W.random_tree(200, rng)
    u, l, d, f = _values(p, rng)
    l = u.copy()
    A = hines_dense(p, u[0], l[0], d[0])
    V, _ = oracle.hines_solve(p, u, l, d, f)
    xr = scipy.linalg.cho_solve(scipy.linalg.cho_factor(A), f[0])
    assert relerr(V, xr) < 1e-14


def test_renumbering_invariance():
    """Any other parent-first numbering of the same tree gives the same
    voltages, permuted."""
    rng = np.random.default_rng(13)
    n = 60
    p = W.random_tree(n, rng)
    u, l, d, f = _values(p, rng)
    # breadth-first order is another numbering with parents first
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[p[i]].append(i)
    order = [0]
    for v in order:
        order.extend(reversed(children[v]))
    new_of = np.empty(n, dtype=np.int64)
    new_of[order] = np.arange(n)
    q = np.full(n, -1, dtype=np.int32)
    for old in range(1, n):
        q[new_of[old]] = new_of[p[old]]
    assert np.all(q[1:] < np.arange(1, n))
    perm = np.array(order)
    V, _ = oracle.hines_solve(p, u, l, d, f)
    V2, _ = oracle.hines_solve(q, u[:, perm], l[:, perm], d[:, perm], f[:, perm])
    np.testing.assert_allclose(V2[0], V[0, perm], rtol=1e-14, atol=1e-15)


def test_multi_equals_one_by_one_and_order_free():
    rng = np.random.default_rng(14)
    hm = W.hines_multi(40, 5, 60, rng=rng)
    V, info = oracle.hines_multi_solve(hm.offsets, hm.parent, hm.u, hm.l, hm.d, hm.rhs)
    assert np.all(info == 0)
    for s in range(hm.batch):
        p, u, l, d, r = hm.neuron(s)
        Vs, _ = oracle.hines_solve(p, u, l, d, r)
        np.testing.assert_array_equal(V[hm.offsets[s]:hm.offsets[s + 1]], Vs[0])
    # reversed neuron order
    rev = list(range(hm.batch))[::-1]
    sizes = hm.sizes[rev]
    off = np.zeros(hm.batch + 1, dtype=np.int64); np.cumsum(sizes, out=off[1:])
    cat = lambda arr: np.concatenate([arr[hm.offsets[s]:hm.offsets[s + 1]] for s in rev])
    V2, _ = oracle.hines_multi_solve(off, cat(hm.parent), cat(hm.u), cat(hm.l), cat(hm.d), cat(hm.rhs))
    np.testing.assert_array_equal(V2, cat(V))


def test_d_input_not_modified_and_info():
    p = np.array([-1, 0, 1, 1], dtype=np.int32)
    rng = np.random.default_rng(1)
    u, l, d, f = _values(p, rng)
    d0 = d.copy()
    oracle.hines_solve(p, u, l, d, f)
    np.testing.assert_array_equal(d, d0)
    dz = d.copy(); dz[0, 3] = 0.0
    _, info = oracle.hines_solve(p, u, l, dz, f)
    assert info[0] == 4                     # compartment 3 is eliminated first
    with pytest.raises(ValueError):
        oracle.hines_solve(np.array([-1, 1, 0], dtype=np.int32), *(np.ones((1, 3)),) * 4)


@pytest.mark.slow
def test_residual_full_workload_mono_and_multi_samples():
    hm = W.hines_mono(512, 64, rng=np.random.default_rng(21))
    fl = [W.to_flat(v) for v in (hm.u, hm.l, hm.d, hm.rhs)]
    V, info = oracle.hines_solve(hm.parent, *fl)
    assert np.all(info == 0)
    for s in range(0, 64, 9):
        A = hines_dense(hm.parent, fl[0][s], fl[1][s], fl[2][s])
        r = A @ V[s] - fl[3][s]
        assert np.max(np.abs(r)) < 1e-14 * np.max(np.abs(A).sum(1)) * np.max(np.abs(V[s]))
    mm = W.hines_multi(6, 256, 2048, rng=np.random.default_rng(22))
    V, info = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    for s in range(mm.batch):
        p, u, l, d, r = mm.neuron(s)
        A = hines_dense(p, u, l, d)
        res = A @ V[mm.offsets[s]:mm.offsets[s + 1]] - r
        assert np.max(np.abs(res)) < 1e-14 * np.max(np.abs(A).sum(1)) * np.max(np.abs(V))
