"""The seeded generators: determinism, shapes and the stated structure."""
import numpy as np

import workloads as W


def test_deterministic_and_shapes():
    a = W.penta_dominant(16, 10)
    b = W.penta_dominant(16, 10)
    for x, y in zip(a.diagonals + (a.f,), b.diagonals + (b.f,)):
        np.testing.assert_array_equal(x, y)
        assert x.shape == (16, 10)


def test_penta_dominance_and_outside_zeros():
    pb = W.penta_dominant(32, 50, rng=np.random.default_rng(0))
    off = np.abs(pb.a) + np.abs(pb.b) + np.abs(pb.d) + np.abs(pb.e)
    assert np.all(pb.c - off >= 1.0)
    assert np.all(pb.a[:2] == 0) and np.all(pb.b[0] == 0)
    assert np.all(pb.d[-1] == 0) and np.all(pb.e[-2:] == 0)
    cy = W.penta_dominant(32, 5, cyclic=True, rng=np.random.default_rng(0))
    assert np.all(cy.a[:2] != 0)


def test_tree_rule_and_stats():
    p = W.random_tree(512, np.random.default_rng(1))
    assert p[0] == -1
    i = np.arange(1, 512)
    assert np.all((p[1:] < i) & (p[1:] >= np.maximum(0, i - 8)))
    st = W.tree_stats(p)
    # the literal parent rule yields about a quarter of branch points
    assert 0.18 < st["branch_frac"] < 0.34
    assert st["max_parent_distance"] <= 8


def test_hines_rows_dominant():
    hm = W.hines_mono(64, 20, rng=np.random.default_rng(2))
    n = 64
    acc = np.abs(hm.l).copy()
    for i in range(1, n):
        acc[hm.parent[i]] += np.abs(hm.u[i])
    assert np.all(hm.d - acc >= 1.0)
    assert np.all(hm.u[0] == 0) and np.all(hm.l[0] == 0)


def test_hines_multi_layout():
    mm = W.hines_multi(30, 5, 40, rng=np.random.default_rng(3))
    assert mm.offsets[-1] == mm.sizes.sum() == len(mm.u)
    assert mm.sizes.min() >= 5 and mm.sizes.max() <= 40
    for s in range(mm.batch):
        p = mm.neuron(s)[0]
        assert p[0] == -1 and np.all(p[1:] < np.arange(1, len(p)))


def test_modes_distinct_wavenumbers():
    ic = W.hyperdiffusion_modes(256, 64)
    assert ic.C0.shape == (256, 64)
    for row in ic.k:
        assert len(set(row.tolist())) == 4 and row.min() >= 1 and row.max() <= 16


def test_tri_dominance_and_outside_zeros():
    tb = W.tri_dominant(33, 20, rng=np.random.default_rng(1), chunk=8)
    assert np.all(tb.a[0] == 0) and np.all(tb.c[-1] == 0)
    assert np.all(tb.b > np.abs(tb.a) + np.abs(tb.c) + 1)
    assert np.all(tb.b < np.abs(tb.a) + np.abs(tb.c) + 2)
    again = W.tri_dominant(33, 20, rng=np.random.default_rng(1), chunk=8)
    np.testing.assert_array_equal(tb.y, again.y)


def test_dfs_tree_is_a_preorder_of_the_drawn_tree():
    """Depth-first numbering: each compartment's parent is the one before it
    or an ancestor of it; the same tree as random_tree's draw up to the
    numbering (children counts agree); parents far back occur."""
    rng = np.random.default_rng(4)
    far = 0
    for n in (1, 2, 3, 17, 300, 2048):
        p = W.dfs_tree(n, np.random.default_rng(n))
        p0 = W.random_tree(n, np.random.default_rng(n))
        assert p[0] == -1 and np.all(p[1:] < np.arange(1, n))
        for i in range(1, n):
            a = i - 1
            while a != p[i] and a > 0:
                a = p[a]
            assert a == p[i]
        kids = lambda q: np.sort(np.bincount(q[1:], minlength=n)) if n > 1 else q
        np.testing.assert_array_equal(kids(p), kids(p0))
        far = max(far, int(np.max(np.arange(1, n) - p[1:], initial=0)))
    assert far > 100
    hm = W.hines_mono(300, 4, rng=rng, dfs=True)
    acc = np.abs(hm.l).copy()
    for i in range(1, 300):
        acc[hm.parent[i]] += np.abs(hm.u[i])
    assert np.all(hm.d - acc >= 1.0)
    assert W.WORKLOADS[11]["dfs"] and W.WORKLOADS[12]["dfs"] and W.WORKLOADS[13]["n"] == 960
