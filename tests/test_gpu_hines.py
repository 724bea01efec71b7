"""GPU parity: Hines solves (mono- and multi-morphology) against the oracle.

Per-neuron normwise relative error <= 1e-10 on identical inputs, through the
C-ABI (plan, pack, solve, unpack).  Covers ragged batches, a single
compartment, chain trees, trees whose parent distance exceeds the on-chip
window (general variant), breakdown reporting, and sampled neurons of the
full mono (100000 x 512) and multi (32768 neurons of 256..2048) workloads.
The small-batch cases run both schedules (one lane per neuron, and the
per-level section schedule that the automatic choice takes for them)."""
import numpy as np
import pytest
import torch

import banded_pde_solvers_amd as bps
import oracle
import workloads as W
from gpu_util import buf, dev, host, info_buf

pytestmark = pytest.mark.gpu


def _rel_per_neuron(x, y, off, skip=()):
    errs = []
    for s in range(len(off) - 1):
        if s in skip:
            continue
        a, b = x[off[s]:off[s + 1]], y[off[s]:off[s + 1]]
        errs.append(np.linalg.norm(a - b) / np.linalg.norm(b))
    return float(np.max(errs))


SCHEDULES = [bps.BPS_HINES_LANES, bps.BPS_HINES_LEVELS]


def _solve_mono(hm, ld=0, schedule=bps.BPS_HINES_AUTO):
    n, batch = hm.u.shape
    plan = bps.hines_plan_create(batch, [n], hm.parent, mono=True, ld=ld, schedule=schedule)
    if schedule != bps.BPS_HINES_AUTO:
        assert plan.uses_levels == (schedule == bps.BPS_HINES_LEVELS)
    ldd = ld or batch
    pad = lambda v: np.pad(v, ((0, 0), (0, ldd - batch)))
    u, l, d, r = (dev(pad(v)) for v in (hm.u, hm.l, hm.d, hm.rhs))
    work = buf(bps.hines_work_bytes(plan))
    info = info_buf(batch)
    bps.hines_solve_batch(plan, u, l, d, r, work, info)
    out = host(r)[:, :batch]
    np.testing.assert_array_equal(host(d)[:, :batch], hm.d)   # d is not modified
    plan.close()
    return out, host(info).astype(int)


def _oracle_mono(hm):
    V, info = oracle.hines_solve(hm.parent, *(W.to_flat(v) for v in (hm.u, hm.l, hm.d, hm.rhs)))
    return W.to_interleaved(V), info


def _cols_err(x, y):
    return float(np.max(np.linalg.norm(x - y, axis=0) / np.linalg.norm(y, axis=0)))


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("n,batch", [(1, 5), (2, 64), (9, 65), (100, 129), (512, 1000)])
def test_mono_matches_oracle(n, batch, schedule):
    print(f"hines mono n={n} batch={batch} schedule={schedule}", flush=True)
    hm = W.hines_mono(n, batch, rng=np.random.default_rng(n + 17 * batch))
    out, info = _solve_mono(hm, schedule=schedule)
    ref, rinfo = _oracle_mono(hm)
    assert _cols_err(out, ref) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_mono_ld_and_chain_tree(schedule):
    rng = np.random.default_rng(4)
    hm = W.hines_mono(300, 70, rng=rng)
    hm.parent = np.arange(-1, 299, dtype=np.int32)          # chain: tridiagonal (Thomas)
    acc = np.abs(hm.l).copy()
    for i in range(1, 300):
        acc[hm.parent[i]] += np.abs(hm.u[i])
    hm.d = acc + 1.0 + rng.uniform(0, 1, hm.d.shape)
    out, _ = _solve_mono(hm, ld=128, schedule=schedule)
    ref, _ = _oracle_mono(hm)
    assert _cols_err(out, ref) <= 1e-10


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_mono_long_parent_distance_general_variant(schedule):
    """Parents up to 200 rows away (beyond the 16-slot on-chip window)."""
    rng = np.random.default_rng(5)
    n, batch = 400, 130
    hm = W.hines_mono(n, batch, rng=rng)
    i = np.arange(1, n)
    hm.parent = np.r_[-1, rng.integers(np.maximum(0, i - 200), i)].astype(np.int32)
    acc = np.abs(hm.l).copy()
    for j in range(1, n):
        acc[hm.parent[j]] += np.abs(hm.u[j])
    hm.d = acc + 1.0 + rng.uniform(0, 1, hm.d.shape)
    assert W.tree_stats(hm.parent)["max_parent_distance"] > 16
    out, info = _solve_mono(hm, schedule=schedule)
    ref, _ = _oracle_mono(hm)
    assert _cols_err(out, ref) <= 1e-10
    assert np.all(info == 0)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("n,batch,ld", [(300, 70, 128), (33, 1, 3), (512, 1000, 1024)])
def test_mono_pack_solve_unpack(n, batch, ld, schedule):
    """The mono layout transform of the Hines page (section 3, done once):
    flat neuron-after-neuron values -> Full-Interleaved [n][ld] with ld >
    batch -> solve -> flat.  The padding columns of every packed array read
    0 (the packed buffers start as NaN), the round trip of an array is
    exact, and every neuron matches the oracle."""
    print(f"hines mono pack n={n} batch={batch} ld={ld} schedule={schedule}", flush=True)
    hm = W.hines_mono(n, batch, rng=np.random.default_rng(n + 3 * ld))
    plan = bps.hines_plan_create(batch, [n], hm.parent, mono=True, ld=ld, schedule=schedule)
    assert plan.elems == n * ld
    flats = [dev(W.to_flat(v).reshape(-1)) for v in (hm.u, hm.l, hm.d, hm.rhs)]
    packed = [torch.full((n, ld), float("nan"), dtype=torch.float64, device="cuda:0")
              for _ in range(4)]
    for f, q in zip(flats, packed):
        bps.hines_pack(plan, f, q)
    for q, v in zip(packed, (hm.u, hm.l, hm.d, hm.rhs)):
        h = host(q)
        np.testing.assert_array_equal(h[:, :batch], v)
        assert np.all(h[:, batch:] == 0.0)
    back = torch.full_like(flats[2], float("nan"))
    bps.hines_unpack(plan, packed[2], back)
    np.testing.assert_array_equal(host(back), host(flats[2]))
    work = buf(bps.hines_work_bytes(plan))
    info = info_buf(batch)
    bps.hines_solve_batch(plan, *packed, work, info)
    out = torch.full_like(flats[3], float("nan"))
    bps.hines_unpack(plan, packed[3], out)
    got = host(out).reshape(batch, n).T
    ref, rinfo = _oracle_mono(hm)
    assert _cols_err(got, ref) <= 1e-10
    np.testing.assert_array_equal(host(info).astype(int), rinfo)
    plan.close()


def _tree_at_distance(n, dist, rng):
    """Parents in the window of 8 rows, with every 29th node's parent planted
    exactly `dist` rows up: the largest parent distance is `dist`."""
    p = W.random_tree(n, rng)
    p[dist::29] = np.arange(dist, n, 29) - dist
    assert W.tree_stats(p)["max_parent_distance"] == dist
    return p


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dist", [16, 17])
def test_mono_parent_distance_window_edge(dist, schedule):
    """Largest parent distance 16 (the last one the 16-slot on-chip window
    of pending updates and recent voltages holds: the child's slot is the
    parent's) and 17 (the first one sent to the global accumulators)."""
    print(f"hines mono window edge dist={dist} schedule={schedule}", flush=True)
    rng = np.random.default_rng(100 + dist)
    hm = _tree_values(_tree_at_distance(200, dist, rng), 130, rng)
    out, info = _solve_mono(hm, schedule=schedule)
    ref, rinfo = _oracle_mono(hm)
    assert _cols_err(out, ref) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)


@pytest.mark.parametrize("schedule", SCHEDULES + [bps.BPS_HINES_SPLIT])
@pytest.mark.parametrize("dist", [16, 17])
def test_multi_parent_distance_window_edge(dist, schedule):
    """As the mono case, for blocks of different trees: every neuron with
    more than `dist` compartments carries parents at exactly `dist`."""
    print(f"hines multi window edge dist={dist} schedule={schedule}", flush=True)
    rng = np.random.default_rng(200 + dist)
    mm = W.hines_multi(150, 10, 90, rng=rng)
    for s in range(mm.batch):
        n = int(mm.sizes[s])
        if n <= dist:
            continue
        o0, o1 = mm.offsets[s], mm.offsets[s + 1]
        p = _tree_at_distance(n, dist, rng)
        mm.parent[o0:o1] = p
        u = mm.u[o0:o1]
        d = 1.0 + np.abs(mm.l[o0:o1]) + rng.uniform(0, 1, n)   # l of the root is 0
        for j in range(1, n):
            d[p[j]] += abs(u[j])
        mm.d[o0:o1] = d
    out, info = _run_multi(mm, schedule)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    assert _rel_per_neuron(out, ref, mm.offsets) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)


def _run_multi(mm, schedule=bps.BPS_HINES_AUTO, min_split=0):
    plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False, schedule=schedule)
    if schedule != bps.BPS_HINES_AUTO:
        assert plan.uses_levels == (schedule == bps.BPS_HINES_LEVELS)
    if schedule in (bps.BPS_HINES_LANES, bps.BPS_HINES_LEVELS):
        assert plan.split == 0
    assert plan.split >= min_split
    E = plan.elems
    packed = [torch.empty(E, dtype=torch.float64, device="cuda:0") for _ in range(4)]
    for src, dst in zip((mm.u, mm.l, mm.d, mm.rhs), packed):
        bps.hines_pack(plan, dev(src), dst)
    work = buf(bps.hines_work_bytes(plan))
    info = info_buf(mm.batch)
    bps.hines_solve_batch(plan, *packed, work, info)
    flat = torch.empty(len(mm.u), dtype=torch.float64, device="cuda:0")
    bps.hines_unpack(plan, packed[3], flat)
    out = host(flat)
    # the packed d is unchanged: unpack it and compare
    dflat = torch.empty_like(flat)
    bps.hines_unpack(plan, packed[2], dflat)
    np.testing.assert_array_equal(host(dflat), mm.d)
    plan.close()
    return out, host(info).astype(int)


@pytest.mark.parametrize("batch,nmin,nmax,schedule",
                         [(1, 1, 1, 1), (3, 1, 7, 1), (70, 5, 60, 1), (200, 256, 2048, 1),
                          (1, 1, 1, 2), (3, 1, 7, 2), (70, 5, 60, 2), (200, 256, 2048, 2),
                          # 1032 blocks: more than one per SIMD, the occupancy-first
                          # kernel configuration; the automatic choice
                          (66000, 2, 9, 0)])
def test_multi_matches_oracle(batch, nmin, nmax, schedule):
    print(f"hines multi batch={batch} n in [{nmin},{nmax}] schedule={schedule}", flush=True)
    mm = W.hines_multi(batch, nmin, nmax, rng=np.random.default_rng(batch + nmax))
    out, info = _run_multi(mm, schedule)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    assert _rel_per_neuron(out, ref, mm.offsets) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)


# ---- trees on two lanes (BPS_HINES_SPLIT, and the automatic choice for
# batches whose largest trees are twice the smallest) ----------------------------

@pytest.mark.parametrize("batch,nmin,nmax", [(1, 600, 600), (5, 32, 40), (130, 20, 700),
                                             (300, 256, 2048),
                                             # one- and two-compartment trees beside split ones
                                             (200, 1, 100),
                                             # more than one block per SIMD: the
                                             # occupancy-first configuration
                                             (70000, 30, 60)])
def test_multi_split_matches_oracle(batch, nmin, nmax):
    print(f"hines multi split batch={batch} n in [{nmin},{nmax}]", flush=True)
    mm = W.hines_multi(batch, nmin, nmax, rng=np.random.default_rng(batch + 7 * nmax))
    out, info = _run_multi(mm, bps.BPS_HINES_SPLIT, min_split=1)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    assert _rel_per_neuron(out, ref, mm.offsets) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)


def test_multi_one_lane_far_parents():
    """One lane per tree (BPS_HINES_LANES) on depth-first numbered trees,
    parents up to thousands of compartments back: far children's updates go
    through the lane's global accumulators; breakdowns near a far parent and
    in a chain, info as Algorithm 1's."""
    print("hines multi one lane, depth-first trees", flush=True)
    rng = np.random.default_rng(61)
    trees = [W.dfs_tree(int(n), rng) for n in rng.integers(20, 3000, size=200)]
    mm = W.hines_multi_trees(trees, rng)
    far = [s for s in range(mm.batch)
           if np.max(np.arange(1, mm.sizes[s]) - mm.neuron(s)[0][1:], initial=0) > 100]
    assert len(far) > 50
    o = mm.offsets
    s1, s2 = far[0], far[1]
    p1 = mm.neuron(s1)[0]
    i1 = int(np.argmax(np.arange(len(p1)) - np.r_[0, p1[1:]]))    # the row with the farthest parent
    mm.u[o[s1]:o[s1 + 1]] = 0.0
    mm.d[o[s1] + int(p1[i1])] = 0.0
    mm.u[o[s2]:o[s2 + 1]] = 0.0
    mm.d[o[s2] + 5] = 0.0
    out, info = _run_multi(mm, bps.BPS_HINES_LANES)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    np.testing.assert_array_equal(info, rinfo)
    assert info[s1] == int(p1[i1]) + 1 and info[s2] == 6
    assert _rel_per_neuron(out, ref, mm.offsets, skip=(s1, s2)) <= 1e-10


def test_multi_split_auto_choice():
    """Two lanes per tree when asked for (every tree whose two-lane schedule
    is shorter); by default, small trees with parents within 16 that fill
    every SIMD with one lane each stay on one lane, and fewer go to the
    separator schedules (which replaced two lanes as the choice there)."""
    print("hines multi split 4096 neurons of 40..210 (parents within 16)", flush=True)
    mm = W.hines_multi(4096, 40, 210, rng=np.random.default_rng(41), window=16)
    assert max(np.max(np.arange(1, n) - mm.neuron(s)[0][1:]) for s, n in enumerate(mm.sizes)) > 8
    plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False, schedule=bps.BPS_HINES_SPLIT)
    assert not plan.uses_levels and not plan.uses_sep
    assert plan.split >= 0.95 * mm.batch
    plan.close()
    out, info = _run_multi(mm, bps.BPS_HINES_SPLIT, min_split=1)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    assert _rel_per_neuron(out, ref, mm.offsets) <= 1e-10
    np.testing.assert_array_equal(info, rinfo)
    # 1025 blocks of one lane per neuron: nothing to fill
    sizes = np.full(1025 * 64, 40, dtype=np.int32)
    rng = np.random.default_rng(42)
    par = np.concatenate([W.random_tree(40, rng) for _ in range(len(sizes))])
    plan = bps.hines_plan_create(len(sizes), sizes, par, mono=False)
    assert not plan.uses_levels and plan.split == 0
    plan.close()
    # 1000 blocks: one lane per tree would leave SIMDs idle: separator schedules
    sizes = np.r_[np.full(1000 * 64 - 2000, 40), np.full(2000, 60)].astype(np.int32)
    par = np.concatenate([W.random_tree(int(n), rng) for n in sizes])
    plan = bps.hines_plan_create(len(sizes), sizes, par, mono=False)
    assert plan.uses_sep and plan.split == 0
    plan.close()


def test_multi_split_breakdown_info():
    """info of a tree on two lanes: 1 + the largest index with a bad pivot
    (the first one Algorithm 1 meets), whichever lane meets it."""
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
    out, info = _run_multi(mm, bps.BPS_HINES_SPLIT, min_split=30)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    np.testing.assert_array_equal(info, rinfo)
    assert info[3] == mm.sizes[3] and info[8] == mm.sizes[8] // 3 + 1 and info[21] == 1
    ok = [s for s in range(mm.batch) if s not in bad]
    offs = mm.offsets
    errs = [np.linalg.norm(out[offs[s]:offs[s + 1]] - ref[offs[s]:offs[s + 1]]) /
            np.linalg.norm(ref[offs[s]:offs[s + 1]]) for s in ok]
    assert max(errs) <= 1e-10


def test_multi_split_pack_contract():
    """hines_pack of a split plan writes every compartment once and 0 to
    every other element; hines_unpack inverts it exactly; solves repeat
    bitwise."""
    mm = W.hines_multi(150, 30, 500, rng=np.random.default_rng(13))
    plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False,
                                 schedule=bps.BPS_HINES_SPLIT)
    assert plan.split > 0
    E = plan.elems
    x = np.random.default_rng(1).uniform(1.0, 2.0, len(mm.u))
    packed = torch.full((E,), -7.0, dtype=torch.float64, device="cuda:0")
    bps.hines_pack(plan, dev(x), packed)
    hp = host(packed)
    assert np.count_nonzero(hp) == len(x)
    assert np.array_equal(np.sort(hp[hp != 0]), np.sort(x))
    back = torch.zeros(len(x), dtype=torch.float64, device="cuda:0")
    bps.hines_unpack(plan, packed, back)
    np.testing.assert_array_equal(host(back), x)
    arrs = []
    for v in (mm.u, mm.l, mm.d, mm.rhs):
        t = torch.empty(E, dtype=torch.float64, device="cuda:0")
        bps.hines_pack(plan, dev(v), t)
        arrs.append(t)
    work = buf(bps.hines_work_bytes(plan))
    r0 = arrs[3].clone()
    bps.hines_solve_batch(plan, *arrs, work)
    first = host(arrs[3])
    arrs[3].copy_(r0)
    bps.hines_solve_batch(plan, *arrs, work)
    np.testing.assert_array_equal(host(arrs[3]), first)
    plan.close()


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_multi_general_variant_and_breakdown(schedule):
    rng = np.random.default_rng(6)
    mm = W.hines_multi(90, 20, 120, rng=rng)
    # give neuron 7 long-range parents, and a zero pivot to neuron 11
    o0, o1 = mm.offsets[7], mm.offsets[8]
    n7 = o1 - o0
    mm.parent[o0 + 1:o1] = rng.integers(0, np.arange(1, n7))
    acc = np.abs(mm.l[o0:o1]).copy()
    for j in range(1, n7):
        acc[mm.parent[o0 + j]] += abs(mm.u[o0 + j])
    mm.d[o0:o1] = acc + 1.0
    z = mm.offsets[11] + mm.sizes[11] - 1
    mm.d[z] = 0.0
    out, info = _run_multi(mm, schedule)
    ref, rinfo = oracle.hines_multi_solve(mm.offsets, mm.parent, mm.u, mm.l, mm.d, mm.rhs)
    np.testing.assert_array_equal(info, rinfo)
    assert info[11] == mm.sizes[11]
    ok = [s for s in range(mm.batch) if s != 11]
    offs = mm.offsets
    errs = [np.linalg.norm(out[offs[s]:offs[s + 1]] - ref[offs[s]:offs[s + 1]]) /
            np.linalg.norm(ref[offs[s]:offs[s + 1]]) for s in ok]
    assert max(errs) <= 1e-10


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_mono_as_multi_agree(schedule):
    hm = W.hines_mono(64, 100, rng=np.random.default_rng(8))
    out_mono, _ = _solve_mono(hm, schedule=schedule)
    sizes = np.full(100, 64, dtype=np.int32)
    off = np.arange(101, dtype=np.int64) * 64
    flat = lambda v: W.to_flat(v).reshape(-1)
    mm = W.HinesMulti(sizes, off, np.tile(hm.parent, 100), flat(hm.u), flat(hm.l), flat(hm.d),
                      flat(hm.rhs))
    out_multi, _ = _run_multi(mm, schedule)
    np.testing.assert_allclose(out_multi, flat(out_mono), rtol=1e-13, atol=1e-15)


@pytest.mark.slow
def test_mono_full_workload_sampled():
    cfg = W.WORKLOADS[3]
    print(f"full hines mono {cfg['n']}x{cfg['batch']}", flush=True)
    hm = W.hines_mono(cfg["n"], cfg["batch"])
    out, info = _solve_mono(hm)
    cols = np.unique(np.r_[0, 63, 64, cfg["batch"] - 1,
                           np.random.default_rng(3).integers(0, cfg["batch"], 200)])
    sub = W.HinesMono(hm.parent, *(v[:, cols] for v in (hm.u, hm.l, hm.d, hm.rhs)))
    ref, _ = _oracle_mono(sub)
    assert _cols_err(out[:, cols], ref) <= 1e-10
    assert np.all(info == 0)


@pytest.mark.slow
def test_multi_full_workload_sampled():
    cfg = W.WORKLOADS[4]
    print(f"full hines multi {cfg['batch']} neurons", flush=True)
    mm = W.hines_multi(cfg["batch"], cfg["nmin"], cfg["nmax"])
    out, info = _run_multi(mm)
    assert np.all(info == 0)
    pick = np.unique(np.r_[0, cfg["batch"] - 1, np.random.default_rng(4).integers(0, cfg["batch"], 150)])
    for s in pick:
        p, u, l, d, r = mm.neuron(s)
        V, _ = oracle.hines_solve(p, u, l, d, r)
        got = out[mm.offsets[s]:mm.offsets[s + 1]]
        assert np.linalg.norm(got - V[0]) / np.linalg.norm(V[0]) <= 1e-10


# ---- the level schedule ---------------------------------------------------------

def _tree_values(p, batch, rng):
    n = len(p)
    u = rng.uniform(-1, 0, (n, batch)); l = rng.uniform(-1, 0, (n, batch))
    u[0] = l[0] = 0.0
    d = 1.0 + np.abs(l) + rng.uniform(0, 1, (n, batch))
    for i in range(1, n):
        d[p[i]] += np.abs(u[i])
    return W.HinesMono(np.asarray(p, dtype=np.int32), u, l, d, rng.uniform(-1, 1, (n, batch)))


@pytest.mark.parametrize("shape", ["star", "uniform", "deep_binary", "big"])
def test_levels_tree_shapes(shape):
    """Shapes that stress the section decomposition: a star (n - 1 sections of
    one node, all updating the root at once), uniformly random parents (long
    distances, few levels), a deep tree of long sections, and a tree of 4096
    compartments (128 KiB of LDS).  Both schedules against the oracle and
    each other."""
    rng = np.random.default_rng(77)
    if shape == "star":
        p = np.r_[-1, np.zeros(299, dtype=int)]
    elif shape == "uniform":
        p = np.r_[-1, rng.integers(0, np.arange(1, 800))]
    elif shape == "deep_binary":
        # sections of 40 nodes; every section's tail has two children
        p = [-1]
        for i in range(1, 1200):
            p.append(i - 1 if i % 40 else (i // 40 - 1) // 2 * 40 + 39 if i >= 80 else 39)
        p = np.array(p)
    else:
        p = W.random_tree(4096, rng, window=8)
    batch = 9 if shape == "big" else 40
    hm = _tree_values(p, batch, rng)
    ref, rinfo = _oracle_mono(hm)
    lv, linfo = _solve_mono(hm, schedule=bps.BPS_HINES_LEVELS)
    ln, _ = _solve_mono(hm, schedule=bps.BPS_HINES_LANES)
    assert _cols_err(lv, ref) <= 1e-10
    assert _cols_err(lv, ln) <= 1e-12
    np.testing.assert_array_equal(linfo, rinfo)


def test_levels_breakdown_info():
    """info of the level schedule: 1 + the largest index with a zero pivot,
    the first one Algorithm 1 meets; a zero root pivot alone gives 1."""
    rng = np.random.default_rng(12)
    hm = W.hines_mono(200, 6, rng=rng)
    hm.d[150, 1] = 0.0          # a node's own pivot (if it is a leaf, d'_150 = d_150)
    hm.d[150, 2] = 0.0
    hm.d[40, 2] = 0.0
    hm.u[1:, 4] = 0.0           # decoupled: every pivot is d itself
    hm.d[0, 4] = 0.0            # the root
    _, info = _solve_mono(hm, schedule=bps.BPS_HINES_LEVELS)
    _, rinfo = _oracle_mono(hm)
    np.testing.assert_array_equal(info, rinfo)
    assert info[4] == 1 and info[0] == 0


def test_levels_auto_choice_and_limits():
    rng = np.random.default_rng(13)
    p = W.random_tree(300, rng)
    # automatic choice for mono trees the sixteen-lane schedule takes
    assert bps.hines_plan_create(2621, [300], p, mono=True).uses_sep
    assert bps.hines_plan_create(30000, [300], p, mono=True).uses_sep
    small = W.random_tree(128, rng)
    assert bps.hines_plan_create(16384, [128], small, mono=True).uses_sep      # 2^21 compartments
    plan = bps.hines_plan_create(16385, [128], small, mono=True)
    assert not plan.uses_sep and not plan.uses_levels
    # mono trees the sixteen-lane schedule does not take (a star: 299
    # one-compartment components): levels for at most 786432 compartments
    star = np.array([-1] + [0] * 299, dtype=np.int32)
    assert not bps.hines_plan_create(2621, [300], star, mono=True).uses_sep
    assert bps.hines_plan_create(2621, [300], star, mono=True).uses_levels
    assert not bps.hines_plan_create(2622, [300], star, mono=True).uses_levels
    big = W.random_tree(5000, rng)
    assert not bps.hines_plan_create(10, [5000], big, mono=True).uses_levels
    # multi-morphology batches the separator schedules are not chosen for
    # (small trees, parents within 16, enough to fill every SIMD with one
    # lane each): levels for at most 393216 compartments
    nb = 1024 * 64
    par6 = np.concatenate([W.random_tree(6, rng, window=16) for _ in range(nb)])
    plan = bps.hines_plan_create(nb, np.full(nb, 6, dtype=np.int32), par6, mono=False)
    assert plan.uses_levels and not plan.uses_sep
    par7 = np.concatenate([W.random_tree(7, rng, window=16) for _ in range(nb)])
    plan = bps.hines_plan_create(nb, np.full(nb, 7, dtype=np.int32), par7, mono=False)
    assert not plan.uses_levels and not plan.uses_sep and plan.split == 0
    with pytest.raises(bps.BpsError):
        bps.hines_plan_create(10, [5000], big, mono=True, schedule=bps.BPS_HINES_LEVELS)


def test_small_batch_workload_full():
    """The benchmarked small batch (512 compartments, 256 neurons): the
    automatic choice is sixteen lanes per neuron; every neuron against the
    oracle, with that schedule and with the level schedule."""
    cfg = W.WORKLOADS[10]
    hm = W.hines_mono(cfg["n"], cfg["batch"], rng=W.rng_for(10))
    plan = bps.hines_plan_create(cfg["batch"], [cfg["n"]], hm.parent, mono=True)
    assert plan.uses_sep
    plan.close()
    ref, _ = _oracle_mono(hm)
    for sched in (bps.BPS_HINES_AUTO, bps.BPS_HINES_LEVELS):
        out, info = _solve_mono(hm, schedule=sched)
        assert _cols_err(out, ref) <= 1e-10
        assert np.all(info == 0)
