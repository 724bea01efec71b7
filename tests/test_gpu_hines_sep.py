"""GPU parity: the separator Hines schedules (BPS_HINES_SEP) against the oracle.

Per-neuron normwise relative error <= 1e-10 through the C-ABI, on ragged
batches (not a multiple of the 16 neurons of a workgroup), ld > batch, both
row counts per lane (16 and 32), chains (every component a path), the
largest trees the schedule takes, breakdowns (info equals Algorithm 1's and
the other neurons are unaffected), repeatability, trees with parents far
back (depth-first numbering, wide windows: ring slots given per lane),
sixty-four lanes per neuron (8 or 4 neurons per workgroup), and sampled
neurons of the full 100000 x 512, 53328 x 960 and depth-first 25600 x 2000
workloads; multi-morphology batches (every tree its own
schedule, the schedule-ordered layout) likewise, with the pack contract and
the full 32768-neuron workload sampled."""
import numpy as np
import pytest
import torch

import banded_pde_solvers_amd as bps
import oracle
import workloads as W
from gpu_util import buf, dev, host, info_buf

pytestmark = pytest.mark.gpu

SEP = bps.BPS_HINES_SEP


def _solve(hm, ld=0, schedule=SEP, twice=False):
    n, batch = hm.u.shape
    plan = bps.hines_plan_create(batch, [n], hm.parent, mono=True, ld=ld, schedule=schedule)
    if schedule == SEP:
        assert plan.uses_sep and not plan.uses_levels
    ldd = ld or batch
    pad = lambda v: np.pad(v, ((0, 0), (0, ldd - batch)), constant_values=7.0)
    u, l, d, r = (dev(pad(v)) for v in (hm.u, hm.l, hm.d, hm.rhs))
    r0 = dev(pad(hm.rhs))
    work = buf(bps.hines_work_bytes(plan))
    info = info_buf(batch)
    bps.hines_solve_batch(plan, u, l, d, r, work, info)
    out = host(r)
    if twice:
        bps.hines_solve_batch(plan, u, l, d, r0, work, info)
        np.testing.assert_array_equal(host(r0), out)          # bitwise repeatable
    np.testing.assert_array_equal(out[:, batch:], pad(hm.rhs)[:, batch:])   # padding untouched
    np.testing.assert_array_equal(host(d)[:, :batch], hm.d)
    plan.close()
    return out[:, :batch], host(info).astype(int)


def _oracle(hm):
    V, info = oracle.hines_solve(hm.parent, *(W.to_flat(v) for v in (hm.u, hm.l, hm.d, hm.rhs)))
    return W.to_interleaved(V), info


def _cols_err(x, y):
    return float(np.max(np.linalg.norm(x - y, axis=0) / np.linalg.norm(y, axis=0)))


def _values(p, batch, rng):
    n = len(p)
    u = rng.uniform(-1, 0, (n, batch))
    l = rng.uniform(-1, 0, (n, batch))
    u[0] = l[0] = 0.0
    d = 1.0 + np.abs(l) + rng.uniform(0, 1, (n, batch))
    for i in range(1, n):
        d[p[i]] += np.abs(u[i])
    return W.HinesMono(np.asarray(p, dtype=np.int32), u, l, d, rng.uniform(-1, 1, (n, batch)))


@pytest.mark.parametrize("n,batch,ld", [(1, 3, 0), (2, 17, 0), (33, 16, 0), (100, 15, 20),
                                        (200, 33, 0), (257, 100, 104), (512, 1000, 0),
                                        (512, 4099, 4160), (530, 77, 0), (600, 33, 40),
                                        (700, 130, 0), (800, 1000, 0), (960, 257, 260)])
def test_sep_matches_oracle(n, batch, ld):
    print(f"hines sep n={n} batch={batch} ld={ld}", flush=True)
    hm = W.hines_mono(n, batch, rng=np.random.default_rng(n + 31 * batch))
    out, info = _solve(hm, ld=ld, twice=(n in (512, 800)))
    ref, rinfo = _oracle(hm)
    assert _cols_err(out, ref) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)
    assert np.all(info == 0)


@pytest.mark.parametrize("shape", ["chain", "far8", "caterpillar", "window2", "broom",
                                   "far9", "window64", "dfs", "comb_reversed"])
def test_sep_tree_shapes(shape):
    rng = np.random.default_rng(5)
    n = 480
    if shape == "chain":
        p = np.r_[-1, np.arange(n - 1)]
    elif shape == "far8":
        p = np.array([-1] + [max(0, i - 8) for i in range(1, n)])
    elif shape == "caterpillar":
        p = np.array([-1] + [i - 2 if i % 2 == 0 else i - 1 for i in range(1, n)])
    elif shape == "window2":
        p = W.random_tree(n, rng, window=2)
    elif shape == "far9":
        p = np.array([-1] + [max(0, i - 9) for i in range(1, n)])
    elif shape == "window64":
        p = W.random_tree(n, rng, window=64)
    elif shape == "dfs":
        p = W.dfs_tree(n, rng)
    elif shape == "comb_reversed":
        # spine 0..k, then its leaves from the last spine compartment back
        p = np.array([-1] + list(range(119)) + list(range(119, -1, -1)))
    else:
        p = np.array([-1] + [max(0, i - 1 - (i - 1) % 8) for i in range(1, n)])
    print(f"hines sep shape={shape}", flush=True)
    hm = _values(p, 50, rng)
    out, info = _solve(hm)
    ref, _ = _oracle(hm)
    assert _cols_err(out, ref) <= 1e-10
    assert np.all(info == 0)


def test_sep_breakdown_info():
    """A neuron with a bad pivot is solved again by Algorithm 1: its info is
    Algorithm 1's; the other neurons of its workgroup are unaffected."""
    rng = np.random.default_rng(12)
    hm = W.hines_mono(300, 40, rng=rng)
    hm.d[299, 1] = 0.0                  # a leaf's pivot is its own d
    hm.d[150, 5] = np.nan               # propagates in every order
    hm.d[0, 9] = np.inf                 # the root
    hm.u[1:, 20] = 0.0                  # decoupled: every pivot is d itself
    hm.d[0, 20] = 0.0
    hm.d[40, 33] = 0.0
    hm.u[1:, 33] = 0.0
    print("hines sep breakdown", flush=True)
    out, info = _solve(hm)
    ref, rinfo = _oracle(hm)
    np.testing.assert_array_equal(info, rinfo)
    assert info[1] == 300 and info[5] == 151 and info[9] == 1 and info[20] == 1 and info[33] == 41
    ok = [s for s in range(hm.u.shape[1]) if s not in (1, 5, 9, 20, 33)]
    assert _cols_err(out[:, ok], ref[:, ok]) <= 1e-10


@pytest.mark.parametrize("n", [600, 1000])
def test_sep_thirty_two_lanes_depth_first(n):
    """Thirty-two lanes per neuron on depth-first numbered trees, a ragged
    batch, with a breakdown in one neuron."""
    print(f"hines sep 32 lanes dfs n={n}", flush=True)
    rng = np.random.default_rng(n)
    hm = _values(W.dfs_tree(n, rng), 70, rng)
    assert bps.hines_sep_schedule(hm.parent)["lanes"] == 32
    hm.d[n // 2, 9] = 0.0
    hm.u[:, 9] = 0.0                      # decoupled: every pivot is d itself
    out, info = _solve(hm)
    ref, rinfo = _oracle(hm)
    np.testing.assert_array_equal(info, rinfo)
    assert info[9] == n // 2 + 1
    ok = [s for s in range(70) if s != 9]
    assert _cols_err(out[:, ok], ref[:, ok]) <= 1e-10


@pytest.mark.parametrize("n,batch,ld,kind,neu", [(1300, 70, 0, "win8", 8), (1500, 1003, 1010, "dfs", 8),
                                                 (2047, 261, 0, "win8", 8), (2047, 130, 0, "dfs", 8),
                                                 (2047, 517, 0, "win16", 4)])
def test_sep_sixty_four_lanes(n, batch, ld, kind, neu):
    """Sixty-four lanes per neuron: 8 neurons per workgroup, or 4 when the
    LDS of 8 does not fit (the workgroups sharing a row segment grouped by
    XCD, a ragged last run), window and depth-first numbered trees, with a
    breakdown in one neuron."""
    print(f"hines sep 64 lanes n={n} batch={batch} ld={ld} {kind}", flush=True)
    if kind == "win16":
        p = W.random_tree(n, np.random.default_rng(10), window=16)
        rng = np.random.default_rng(n + batch)
    else:
        rng = np.random.default_rng(n + batch)
        p = W.dfs_tree(n, rng) if kind == "dfs" else W.random_tree(n, rng)
    hm = _values(p, batch, rng)
    S = bps.hines_sep_schedule(hm.parent)
    assert S["lanes"] == 64 and S["neurons"] == neu
    hm.d[n // 3, 5] = 0.0
    hm.u[:, 5] = 0.0                      # decoupled: every pivot is d itself
    out, info = _solve(hm, ld=ld, twice=(batch == 130))
    ref, rinfo = _oracle(hm)
    np.testing.assert_array_equal(info, rinfo)
    assert info[5] == n // 3 + 1
    ok = [s for s in range(batch) if s != 5]
    assert _cols_err(out[:, ok], ref[:, ok]) <= 1e-10


def _kind_tree(kind, n, rng):
    if kind == 0:
        return W.random_tree(n, rng, window=int(rng.integers(1, 65)))
    if kind == 1:
        return W.dfs_tree(n, rng, window=int(rng.integers(1, 17)))
    p = np.empty(n, dtype=np.int32)           # bushy: parent uniform over all before
    p[0] = -1
    for i in range(1, n):
        p[i] = rng.integers(0, i)
    return p


def test_sep_fuzz_mono_and_multi():
    """Seeded trees of every kind (windows 1..64, depth-first, bushy), mono
    plans the schedule takes and one multi-morphology batch of them all,
    against the oracle."""
    rng = np.random.default_rng(4242)
    done = 0
    for it in range(12):
        n = int(rng.integers(2, 2048))
        p = _kind_tree(it % 3, n, rng)
        if bps.hines_sep_schedule(p) is None:
            continue
        print(f"hines sep fuzz mono it={it} n={n}", flush=True)
        hm = _values(p, 37, rng)
        out, info = _solve(hm)
        ref, rinfo = _oracle(hm)
        assert _cols_err(out, ref) <= 1e-10, (it, n)
        np.testing.assert_array_equal(info, rinfo)
        done += 1
    assert done >= 6
    print("hines sep fuzz multi", flush=True)
    trees = [_kind_tree(k % 3, int(rng.integers(1, 1500)), rng) for k in range(300)]
    mm = W.hines_multi_trees(trees, rng)
    out, info = _run_multi(mm)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    assert _multi_err(mm, out, ref) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)


def test_sep_refusals_and_auto():
    rng = np.random.default_rng(3)
    # trees with parents far back are taken (ring slots per lane), also by
    # the automatic choice
    for p in (W.random_tree(300, rng, window=16), W.dfs_tree(300, rng)):
        assert (np.arange(1, 300) - p[1:]).max() > 8
        bps.hines_plan_create(64, [300], p, mono=True, schedule=SEP).close()
        plan = bps.hines_plan_create(64, [300], p, mono=True)
        assert plan.uses_sep
        plan.close()
    # trees of 1300..2047 on sixty-four lanes; by the automatic choice with
    # parents far back, or in batches below 24576 neurons (one lane per
    # neuron is faster for larger batches of trees with parents within 16)
    for p, far in ((W.random_tree(1500, rng), False), (W.dfs_tree(1500, rng), True)):
        bps.hines_plan_create(64, [1500], p, mono=True, schedule=SEP).close()
        for batch in (4096, 24575, 24576, 32768):
            plan = bps.hines_plan_create(batch, [1500], p, mono=True)
            assert plan.uses_sep == (far or batch < 24576) and not plan.uses_levels, batch
            plan.close()
    # 32 lanes of 32 rows: taken with at most 32 separators, left to one lane
    # per neuron beyond (parents within 16, 24576 neurons or more)
    seen = set()
    for seed in range(40):
        p = W.random_tree(1024, np.random.default_rng(seed))
        S = bps.hines_sep_schedule(p)
        if S is None or S["lanes"] != 32 or S["R"] != 32:
            continue
        squeezed = S["ns"] > 32
        plan = bps.hines_plan_create(32768, [1024], p, mono=True)
        assert plan.uses_sep == (not squeezed), (seed, S["ns"])
        plan.close()
        plan = bps.hines_plan_create(4096, [1024], p, mono=True)
        assert plan.uses_sep, (seed, S["ns"])
        plan.close()
        seen.add(squeezed)
        if len(seen) == 2:
            break
    assert seen == {True, False}
    # above the 2047 compartments of the row codes; a star of 1499 components
    with pytest.raises(bps.BpsError):
        bps.hines_plan_create(64, [2048], W.random_tree(2048, rng), mono=True, schedule=SEP)
    with pytest.raises(bps.BpsError):
        bps.hines_plan_create(64, [1500], np.array([-1] + [0] * 1499, dtype=np.int32), mono=True,
                              schedule=SEP)
    # a multi-morphology tree too large for 128 lanes of 32 rows
    sizes = np.array([50, 50, 9000], dtype=np.int32)
    with pytest.raises(bps.BpsError):
        bps.hines_plan_create(3, sizes, np.concatenate([W.random_tree(50, rng)] * 2 +
                                                       [W.random_tree(9000, rng)]), mono=False, schedule=SEP)


@pytest.mark.slow
@pytest.mark.parametrize("which", [3, 13, 14])
def test_sep_full_workload_sampled(which):
    """The full mono workloads on sixteen, thirty-two and sixty-four lanes
    per neuron (the benchmark's inputs and launch), sampled neurons against
    the oracle."""
    cfg = W.WORKLOADS[which]
    print(f"full hines mono {cfg['n']}x{cfg['batch']} sep (workload {which})", flush=True)
    hm = W.hines_mono(cfg["n"], cfg["batch"], rng=W.rng_for(which), dfs=cfg.get("dfs", False))
    S = bps.hines_sep_schedule(hm.parent)
    assert S["lanes"] == {3: 16, 13: 32, 14: 64}[which]
    out, info = _solve(hm)
    cols = np.unique(np.r_[0, 7, 8, 15, 16, cfg["batch"] - 1,
                           np.random.default_rng(which).integers(0, cfg["batch"], 200)])
    sub = W.HinesMono(hm.parent, *(v[:, cols] for v in (hm.u, hm.l, hm.d, hm.rhs)))
    ref, _ = _oracle(sub)
    assert _cols_err(out[:, cols], ref) <= 1e-10
    assert np.all(info == 0)


# ---- multi-morphology: every tree its own schedule -------------------------------

def _run_multi(mm, schedule=SEP, twice=False):
    plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False, schedule=schedule)
    if schedule == SEP:
        assert plan.uses_sep and not plan.uses_levels and plan.split == 0
    E = plan.elems
    packed = [torch.empty(E, dtype=torch.float64, device="cuda:0") for _ in range(4)]
    for src, dst in zip((mm.u, mm.l, mm.d, mm.rhs), packed):
        bps.hines_pack(plan, dev(src), dst)
    r0 = packed[3].clone()
    work = buf(bps.hines_work_bytes(plan))
    info = info_buf(mm.batch)
    bps.hines_solve_batch(plan, *packed, work, info)
    if twice:
        bps.hines_solve_batch(plan, *packed[:3], r0, work, info)
        np.testing.assert_array_equal(host(r0), host(packed[3]))          # bitwise repeatable
    flat = torch.empty(len(mm.u), dtype=torch.float64, device="cuda:0")
    bps.hines_unpack(plan, packed[3], flat)
    out = host(flat)
    dflat = torch.empty_like(flat)
    bps.hines_unpack(plan, packed[2], dflat)
    np.testing.assert_array_equal(host(dflat), mm.d)
    plan.close()
    return out, host(info).astype(int)


def _multi_err(mm, out, ref, skip=()):
    o = mm.offsets
    return max(np.linalg.norm(out[o[s]:o[s + 1]] - ref[o[s]:o[s + 1]]) / np.linalg.norm(ref[o[s]:o[s + 1]])
               for s in range(mm.batch) if s not in skip)


@pytest.mark.parametrize("batch,nmin,nmax", [(1, 1, 1), (3, 2, 40), (40, 30, 300), (300, 256, 2048),
                                             (5000, 1, 100), (70000, 30, 60)])
def test_sep_multi_matches_oracle(batch, nmin, nmax):
    print(f"hines sep multi batch={batch} n={nmin}..{nmax}", flush=True)
    mm = W.hines_multi(batch, nmin, nmax, rng=np.random.default_rng(batch + nmax))
    out, info = _run_multi(mm, twice=(batch == 300))
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    assert _multi_err(mm, out, ref) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)


def test_sep_multi_many_separators():
    """Trees of doubling chains put more separators than lanes in a workgroup
    (each substitution lane then holds a second one), mixed with random trees."""
    print("hines sep multi: doubling-chain trees", flush=True)
    rng = np.random.default_rng(23)
    trees = [W.doubling_tree(34)] * 40 + [W.doubling_tree(30)] * 9 + \
            [W.random_tree(int(n), rng) for n in rng.integers(200, 900, size=25)]
    mm = W.hines_multi_trees(trees, rng)
    Lo = bps.hines_sep_multi_layout(mm.sizes, mm.parent)
    assert max(int(Lo["tabs"][Lo["wgoff"][w] + 1]) for w in range(Lo["nwg"])) > Lo["K"]
    out, info = _run_multi(mm, twice=True)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    assert _multi_err(mm, out, ref) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)


def test_sep_multi_breakdown_info():
    rng = np.random.default_rng(12)
    mm = W.hines_multi(40, 200, 400, rng=rng)
    bad = {3: "zero_leaf", 8: "nan_mid", 21: "inf_root"}
    for s, kind in bad.items():
        o0, n = mm.offsets[s], int(mm.sizes[s])
        if kind == "zero_leaf":
            mm.d[o0 + n - 1] = 0.0
        elif kind == "nan_mid":
            mm.d[o0 + n // 3] = np.nan
        else:
            mm.d[o0] = np.inf
    print("hines sep multi breakdown", flush=True)
    out, info = _run_multi(mm)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    np.testing.assert_array_equal(info, rinfo)
    assert info[3] == mm.sizes[3] and info[8] == mm.sizes[8] // 3 + 1 and info[21] == 1
    assert _multi_err(mm, out, ref, skip=bad) <= 1e-10


def test_sep_multi_pack_contract():
    """hines_pack writes every compartment once and 0 to every other element;
    hines_unpack inverts it exactly."""
    mm = W.hines_multi(150, 30, 500, rng=np.random.default_rng(13))
    plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False, schedule=SEP)
    packed = torch.empty(plan.elems, dtype=torch.float64, device="cuda:0")
    x = np.arange(1, len(mm.u) + 1, dtype=np.float64)
    bps.hines_pack(plan, dev(x), packed)
    pk = host(packed)
    assert np.count_nonzero(pk) == len(x) and np.array_equal(np.sort(pk[pk != 0]), x)
    back = torch.empty(len(x), dtype=torch.float64, device="cuda:0")
    bps.hines_unpack(plan, packed, back)
    np.testing.assert_array_equal(host(back), x)
    plan.close()


@pytest.mark.slow
def test_sep_multi_full_workload_sampled():
    cfg = W.WORKLOADS[4]
    print(f"full hines multi {cfg['batch']} neurons sep", flush=True)
    mm = W.hines_multi(cfg["batch"], cfg["nmin"], cfg["nmax"])
    out, info = _run_multi(mm)
    assert np.all(info == 0)
    pick = np.unique(np.r_[0, cfg["batch"] - 1, np.random.default_rng(4).integers(0, cfg["batch"], 150)])
    for s in pick:
        p, u, l, d, r = mm.neuron(s)
        V, _ = oracle.hines_solve(p, u, l, d, r)
        got = out[mm.offsets[s]:mm.offsets[s + 1]]
        assert np.linalg.norm(got - V[0]) / np.linalg.norm(V[0]) <= 1e-10


def test_sep_multi_far_parents():
    """Depth-first numbered trees of 256..2048 compartments (parents far
    back), on the automatic choice: separator schedules, against the oracle."""
    print("hines sep multi: depth-first numbered trees", flush=True)
    rng = np.random.default_rng(31)
    trees = [W.dfs_tree(int(n), rng) for n in rng.integers(256, 2049, size=600)] + \
            [W.random_tree(int(n), rng, window=32) for n in rng.integers(256, 2049, size=100)]
    mm = W.hines_multi_trees(trees, rng)
    plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False)
    assert plan.uses_sep and not plan.uses_levels and plan.split == 0
    plan.close()
    out, info = _run_multi(mm, twice=True)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    assert _multi_err(mm, out, ref) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)


def test_sep_multi_hybrid_trees_too_large():
    """A batch whose few trees do not fit a workgroup (6000 and 9000
    compartments, one of 5000 numbered depth first): the automatic choice
    keeps the others on separator schedules and solves those on one lane
    each (after the separators' elements of the layout); pack, solve,
    unpack and info against the oracle, with a breakdown in a large tree and
    in a separator-scheduled one."""
    print("hines sep multi: hybrid with trees too large for a workgroup", flush=True)
    rng = np.random.default_rng(77)
    trees = [W.dfs_tree(int(n), rng) for n in rng.integers(256, 2049, size=300)]
    trees[17] = W.random_tree(6000, rng)
    trees[150] = W.random_tree(9000, rng)
    trees[299] = W.dfs_tree(5000, rng)
    mm = W.hines_multi_trees(trees, rng)
    o = mm.offsets
    for s_, i_ in ((150, 4000), (40, 100)):       # zero pivots, the tree's rows decoupled
        mm.u[o[s_]:o[s_ + 1]] = 0.0
        mm.d[o[s_] + i_] = 0.0
    plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False)
    assert plan.uses_sep and plan.elems > 0
    plan.close()
    out, info = _run_multi(mm, schedule=bps.BPS_HINES_AUTO, twice=True)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    np.testing.assert_array_equal(info, rinfo)
    assert info[150] == 4001 and info[40] == 101
    assert _multi_err(mm, out, ref, skip=(150, 40)) <= 1e-10
    with pytest.raises(bps.BpsError):                 # asked for explicitly: all trees or none
        bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False, schedule=SEP)


def test_sep_multi_auto_choice():
    """The automatic choice for multi-morphology batches: separator schedules
    unless the trees average under 128 compartments, have their parents
    within 16 and are enough (1024 blocks of 64) to fill every SIMD with one
    lane per tree; then one lane per tree."""
    rng = np.random.default_rng(23)
    mm = W.hines_multi(300, 100, 160, rng=rng)
    plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False)
    assert plan.uses_sep                              # 5 blocks: one lane per tree would not fill
    plan.close()
    big = W.hines_multi(64, 256, 2048, rng=rng)
    plan = bps.hines_plan_create(big.batch, big.sizes, big.parent, mono=False)
    assert plan.uses_sep and not plan.uses_levels and plan.split == 0
    plan.close()
    small = W.hines_multi(64, 30, 60, rng=rng)
    plan = bps.hines_plan_create(small.batch, small.sizes, small.parent, mono=False)
    assert plan.uses_sep
    plan.close()
    many = W.hines_multi(1024 * 64, 30, 60, rng=rng)  # fills every SIMD, parents within 8
    plan = bps.hines_plan_create(many.batch, many.sizes, many.parent, mono=False)
    assert not plan.uses_sep and not plan.uses_levels and plan.split == 0
    plan.close()
    far = W.hines_multi_trees([W.dfs_tree(int(n), rng) for n in rng.integers(30, 61, size=1024 * 64)], rng)
    plan = bps.hines_plan_create(far.batch, far.sizes, far.parent, mono=False)
    assert plan.uses_sep                              # the other kernels' general variant otherwise
    plan.close()
    w16 = W.hines_multi(64, 256, 2048, rng=rng, window=16)
    plan = bps.hines_plan_create(w16.batch, w16.sizes, w16.parent, mono=False)
    assert plan.uses_sep
    plan.close()
    out, info = _run_multi(big, schedule=bps.BPS_HINES_AUTO)
    ref, rinfo = oracle.hines_multi_solve(big.offsets, big.parent, big.u, big.l, big.d, big.rhs)
    assert _multi_err(big, out, ref) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)
