"""Host-side checks of the multi-morphology BPS_HINES_SEP layout.

The library's layout of a batch (hines_sep_multi_layout, host only) is run
through a plain Python replay of the kernel: per workgroup, every lane's
first sweep over its steps (values read at (w R + t) K + k, K lanes per
workgroup), the
separators' rows assembled, Algorithm 1 on each tree's separators, the
components' parent voltages, the second sweep; the voltages, mapped back
through the element map, are compared with the oracle tree by tree.  Every
table index the kernel follows is checked against its range first, so a
layout that would send the kernel outside its LDS arrays fails here.
"""
import numpy as np
import pytest

import oracle
import workloads as W

bps = pytest.importorskip("banded_pde_solvers_amd")

LIVE, PATH, PATH0, TOP, SEPR = 1 << 6, 1 << 7, 1 << 8, 1 << 9, 1 << 10


def _lib_or_skip():
    try:
        bps.load_library()
    except bps.BpsLibraryMissing:
        pytest.skip("libbps.so not built")


def _tables(Lo, w):
    wt = Lo["tabs"][Lo["wgoff"][w]:Lo["wgoff"][w + 1]]
    nt, ns, nc, npc, nh, n16 = (int(v) for v in wt[:6])
    trees = wt[8:8 + nt * 5].reshape(nt, 5)
    t16 = wt[8 + nt * 5:].view(np.int16)[:n16].astype(np.int64)
    septab = t16[:ns * 4].reshape(ns, 4)
    comptab = t16[ns * 4:ns * 4 + nc * 3].reshape(nc, 3)
    clist = t16[ns * 4 + nc * 3:ns * 4 + nc * 4]
    return nt, ns, nc, npc, nh, trees, septab, comptab, clist


def _check_ranges(Lo, sizes):
    R, nwg, K = Lo["R"], Lo["nwg"], Lo["K"]
    assert Lo["lds"] <= 40 * 1024 and K == 128
    comp = Lo["comp"]
    total = int(np.sum(sizes))
    live = comp >= 0
    assert np.array_equal(np.sort(comp[live]), np.arange(total))      # every compartment once
    assert np.array_equal(comp[Lo["pos"]], np.arange(total))
    code = Lo["code"].astype(np.int64)
    assert np.all(((code & (LIVE | SEPR)) != 0) == live)
    for w in range(nwg):
        nt, ns, nc, npc, nh, trees, septab, comptab, clist = _tables(Lo, w)
        assert 1 <= nt <= K
        lanes = trees[:, 3] - trees[:, 2]
        assert trees[0, 2] == 0 and np.all(trees[1:, 2] == trees[:-1, 3]) and trees[-1, 3] <= K
        assert trees[0, 0] == 0 and np.all(trees[1:, 0] == trees[:-1, 1]) and trees[-1, 1] == ns
        assert np.all(lanes >= 1)
        for tt in range(nt):
            s0, s1 = trees[tt, 0], trees[tt, 1]
            rp = septab[s0:s1, 0]
            assert np.all((rp == -1) | ((rp > np.arange(s0, s1)) & (rp < s1)))
        assert np.all((septab[:, 1] >= -1) & (septab[:, 1] < nc))
        assert np.all((0 <= septab[:, 2]) & (septab[:, 2] <= septab[:, 3]) & (septab[:, 3] <= nc))
        assert np.all((clist >= 0) & (clist < nc))
        assert np.all((comptab[:, :2] >= -1) & (comptab[:, :2] < ns))
        assert np.all((comptab[:, 2] >= -1) & (comptab[:, 2] < npc))
        lt = Lo["lanetab"][w * K:(w + 1) * K]
        used = lt[:, 0] >= 0
        assert used.sum() == lanes.sum() and np.all(lt[~used, 0] == -1)
        cw = code[w * R * K:(w + 1) * R * K].reshape(R, K)
        # counters of each lane stay inside the workgroup's numbering
        for k in np.flatnonzero(used):
            c = cw[:, k]
            assert lt[k, 1] + ((c & TOP) != 0).sum() <= nc
            assert lt[k, 2] + ((c & PATH) != 0).sum() <= nh
            assert lt[k, 3] + (((c & TOP) != 0) & ((c & PATH) != 0)).sum() <= npc
            assert lt[k, 4] + ((c & SEPR) != 0).sum() <= ns


def _replay(Lo, sizes, u, l, d, rhs):
    R, nwg, comp, K = Lo["R"], Lo["nwg"], Lo["comp"], Lo["K"]
    pk = lambda v: np.where(comp >= 0, v[np.maximum(comp, 0)], 0.0)
    U, Lv, Dv, Rv = pk(u), pk(l), pk(d), pk(rhs)
    out = np.zeros_like(Rv)
    code = Lo["code"].astype(np.int64)
    bad_trees = set()
    with np.errstate(all="ignore"):
        for w in range(nwg):
            nt, ns, nc, npc, nh, trees, septab, comptab, clist = _tables(Lo, w)
            red = np.zeros((nc, 2))
            pdat = np.zeros((npc, 4))
            sepv = np.zeros((ns, 4))
            su = np.zeros(ns)
            hbuf = np.zeros(nh + 2)
            badf = np.zeros(K, dtype=bool)
            q = np.zeros((K, R))
            m = np.zeros((K, R))
            ends = np.zeros((K, 3), dtype=np.int64)
            lt = Lo["lanetab"][w * K:(w + 1) * K]
            for k in range(K):
                tslot, ccomp, chidx, cpidx, csep = (int(v) for v in lt[k])
                ring = np.zeros((8, 2))
                g = P = al = ga = 0.0
                for t in range(R):
                    e = (w * R + t) * K + k
                    c = int(code[e])
                    live = bool(c & LIVE)
                    own, par = c & 7, (c >> 3) & 7
                    u_, l_, d_, r_ = (U[e], Lv[e], Dv[e], Rv[e]) if c & (LIVE | SEPR) else (0, 0, 0, 0)
                    if c & SEPR:
                        sepv[csep] = (d_, r_, l_, u_)
                        su[csep] = u_
                        csep += 1
                    pd = ring[own].copy()
                    po = ring[par].copy()
                    ring[own] = 0.0
                    dd, rr = d_ - pd[0], r_ - pd[1]
                    badf[k] |= live and not (dd != 0.0 and np.isfinite(dd))
                    rcp = 1.0 / dd
                    q[k, t], m[k, t] = rr * rcp, l_ * rcp
                    fac = u_ * rcp
                    if c & PATH0:
                        g, P, al, ga = 1.0, 1.0, 0.0, 0.0
                    h = g * rcp
                    if c & PATH:
                        hbuf[chidx] = h
                        chidx += 1
                        al += P * q[k, t]
                        ga -= P * h
                        P = -m[k, t] * P
                        g = -fac * g
                    cb = np.array([fac * l_, fac * rr]) if live else np.zeros(2)
                    if c & TOP:
                        red[ccomp] = cb
                        ccomp += 1
                        if c & PATH:
                            pdat[cpidx] = (g, al, P, ga)
                            cpidx += 1
                    else:
                        ring[par] = (np.zeros(2) if par == own else po) + cb
                ends[k] = ccomp, chidx, csep
            for i in range(ns):
                rp, pc, cb_, ce = (int(v) for v in septab[i])
                dh, rh, l_, u_ = sepv[i]
                lh = uh = 0.0
                for c in clist[cb_:ce]:
                    dh -= red[c, 0]
                    rh -= red[c, 1]
                if pc >= 0:
                    ut, a_, b_, gm = pdat[comptab[pc, 2]]
                    dh += l_ * u_ * gm
                    rh -= l_ * a_
                    lh, uh = l_ * b_, u_ * ut
                elif rp >= 0:
                    lh, uh = l_, u_
                sepv[i] = (dh, rh, lh, uh)
            tflag = np.zeros(nt, dtype=bool)
            for tt in range(nt):
                s0, s1, l0, l1, T = (int(v) for v in trees[tt])
                anyb = bool(badf[l0:l1].any())
                for i in range(s0, s1):
                    rp = int(septab[i, 0])
                    dh, rh, lh, uh = sepv[i]
                    anyb |= not (dh != 0.0 and np.isfinite(dh))
                    sepv[i, 2:] = rh / dh, lh / dh
                    if rp >= 0:
                        f = uh / dh
                        sepv[rp, 0] -= f * lh
                        sepv[rp, 1] -= f * rh
                tflag[tt] = anyb
                if anyb:
                    bad_trees.add(T)
            # substitution by pointer jumping over the workgroup's separators:
            # x_i = a_i + b_i x_p(i), the header's number of rounds
            rounds = int(Lo["tabs"][Lo["wgoff"][w] + 6])
            a, b, ptr = sepv[:, 2].copy(), -sepv[:, 3], septab[:, 0].copy()
            for k in range(rounds):
                assert k == 0 or np.any(ptr >= 0)           # no round more than needed
                has = ptr >= 0
                pp = np.where(has, ptr, 0)
                a = np.where(has, b * a[pp] + a, a)
                b = np.where(has, b * b[pp], b)
                ptr = np.where(has, ptr[pp], ptr)
            assert np.all(ptr < 0)                          # enough rounds
            sepv[:, 0] = a
            for c in range(nc):
                pc, sc = int(comptab[c, 0]), int(comptab[c, 1])
                red[c] = (sepv[pc, 0] if pc >= 0 else 0.0, su[sc] * sepv[sc, 0] if sc >= 0 else 0.0)
            for k in range(K):
                ccomp, chidx, csep = (int(v) for v in ends[k])
                ring = np.zeros(8)
                sg = 0.0
                for t in range(R - 1, -1, -1):
                    e = (w * R + t) * K + k
                    c = int(code[e])
                    own, par = c & 7, (c >> 3) & 7
                    if c & TOP:
                        ccomp -= 1
                    if c & PATH:
                        chidx -= 1
                    if c & SEPR:
                        csep -= 1
                    xp, s2 = red[ccomp] if c & TOP else (ring[par], None)
                    if c & TOP:
                        sg = s2
                    h = hbuf[chidx] if c & PATH else 0.0
                    x = q[k, t] - m[k, t] * xp - h * sg
                    ring[own] = x
                    if c & SEPR:
                        x = sepv[csep, 0]
                    if c & (LIVE | SEPR):
                        out[e] = x
    V = np.zeros(int(np.sum(sizes)))
    V[comp[comp >= 0]] = out[comp >= 0]
    return V, bad_trees


@pytest.mark.parametrize("batch,nmin,nmax,seed", [(1, 1, 1, 0), (3, 2, 40, 1), (40, 30, 300, 2),
                                                   (70, 256, 2048, 3), (300, 20, 200, 4)])
def test_sep_multi_replay_matches_oracle(batch, nmin, nmax, seed):
    _lib_or_skip()
    mm = W.hines_multi(batch, nmin, nmax, rng=np.random.default_rng(seed))
    Lo = bps.hines_sep_multi_layout(mm.sizes, mm.parent)
    assert Lo is not None
    _check_ranges(Lo, mm.sizes)
    V, bad = _replay(Lo, mm.sizes, mm.u, mm.l, mm.d, mm.rhs)
    assert not bad
    ref, info = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    assert np.all(info == 0)
    o = mm.offsets
    err = max(np.linalg.norm(V[o[s]:o[s + 1]] - ref[o[s]:o[s + 1]]) / np.linalg.norm(ref[o[s]:o[s + 1]])
              for s in range(batch))
    assert err <= 1e-13


def test_sep_multi_replay_far_parents():
    """Depth-first numbered trees and wide windows: parents far back."""
    _lib_or_skip()
    rng = np.random.default_rng(29)
    trees = [W.dfs_tree(int(n), rng) for n in rng.integers(100, 1500, size=30)] + \
            [W.random_tree(int(n), rng, window=40) for n in rng.integers(100, 800, size=10)]
    mm = W.hines_multi_trees(trees, rng)
    assert max(int(np.max(np.arange(1, n) - mm.neuron(s)[0][1:])) for s, n in enumerate(mm.sizes)) > 100
    Lo = bps.hines_sep_multi_layout(mm.sizes, mm.parent)
    assert Lo is not None
    _check_ranges(Lo, mm.sizes)
    V, bad = _replay(Lo, mm.sizes, mm.u, mm.l, mm.d, mm.rhs)
    assert not bad
    ref, info = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    o = mm.offsets
    err = max(np.linalg.norm(V[o[s]:o[s + 1]] - ref[o[s]:o[s + 1]]) / np.linalg.norm(ref[o[s]:o[s + 1]])
              for s in range(mm.batch))
    assert err <= 1e-13


def test_sep_multi_replay_many_separators():
    """Trees of doubling chains give workgroups of more separators than lanes
    (the substitution's lanes then hold a second separator each)."""
    _lib_or_skip()
    mm = W.hines_multi_trees([W.doubling_tree(34)] * 8 + [W.doubling_tree(30)] * 2,
                             np.random.default_rng(17))
    Lo = bps.hines_sep_multi_layout(mm.sizes, mm.parent)
    assert Lo is not None
    assert max(int(Lo["tabs"][Lo["wgoff"][w] + 1]) for w in range(Lo["nwg"])) > Lo["K"]
    _check_ranges(Lo, mm.sizes)
    V, bad = _replay(Lo, mm.sizes, mm.u, mm.l, mm.d, mm.rhs)
    assert not bad
    ref, info = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    o = mm.offsets
    err = max(np.linalg.norm(V[o[s]:o[s + 1]] - ref[o[s]:o[s + 1]]) / np.linalg.norm(ref[o[s]:o[s + 1]])
              for s in range(mm.batch))
    assert err <= 1e-13


@pytest.mark.parametrize("batch,nmin,nmax,window", [(2000, 100, 300, 2), (2000, 30, 2047, 1),
                                                     (3000, 20, 200, 8)])
def test_sep_multi_layout_lds_budget(batch, nmin, nmax, window):
    """Batches whose workgroups fill the LDS budget (many path rows): every
    workgroup within 40 KB, so that four fit in a CU's 160 KB, and every table
    index in range."""
    _lib_or_skip()
    mm = W.hines_multi(batch, nmin, nmax, rng=np.random.default_rng(5), window=window)
    Lo = bps.hines_sep_multi_layout(mm.sizes, mm.parent)
    assert Lo is not None
    assert 4 * Lo["lds"] <= 160 * 1024
    _check_ranges(Lo, mm.sizes)


def test_sep_multi_layout_refusals():
    _lib_or_skip()
    big = W.random_tree(9000, np.random.default_rng(1))
    good = W.random_tree(40, np.random.default_rng(1))
    assert bps.hines_sep_multi_layout([40, 9000], np.r_[good, big]) is None
    assert "too large" in bps.bps_last_error()
    with pytest.raises(bps.BpsError):
        bps.hines_sep_multi_layout([3], [-1, 0, 5])


def test_sep_multi_replay_fuzz():
    """A batch of trees of every kind (windows 1..64, depth-first, bushy
    random recursive trees): the layout replays to the oracle's voltages."""
    _lib_or_skip()
    rng = np.random.default_rng(77)
    trees = []
    for it in range(60):
        n = int(rng.integers(1, 1500))
        if it % 3 == 0:
            trees.append(W.random_tree(n, rng, window=int(rng.integers(1, 65))))
        elif it % 3 == 1:
            trees.append(W.dfs_tree(n, rng, window=int(rng.integers(1, 17))))
        else:
            p = np.empty(n, dtype=np.int32)
            p[0] = -1
            for i in range(1, n):
                p[i] = rng.integers(0, i)
            trees.append(p)
    mm = W.hines_multi_trees(trees, rng)
    Lo = bps.hines_sep_multi_layout(mm.sizes, mm.parent)
    assert Lo is not None
    _check_ranges(Lo, mm.sizes)
    V, bad = _replay(Lo, mm.sizes, mm.u, mm.l, mm.d, mm.rhs)
    assert not bad
    ref, info = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    o = mm.offsets
    err = max(np.linalg.norm(V[o[s]:o[s + 1]] - ref[o[s]:o[s + 1]]) / np.linalg.norm(ref[o[s]:o[s + 1]])
              for s in range(mm.batch))
    assert err <= 1e-13
