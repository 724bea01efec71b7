"""Host-side checks of the two-lane Hines schedule (BPS_HINES_SPLIT).

The library's schedule of one tree (hines_split_schedule, host only) is run
through a plain Python replay of what the two-lane kernel does with it (slot
reads, clears and adds of the first sweep, slot and register reads of the
second, lane by lane in lockstep), and the voltages are compared with the
oracle's Algorithm 1 on the same tree.  A schedule that sent an update to a
wrong slot, or let a slot be reused too early, gives wrong voltages here.
"""
import numpy as np
import pytest

import oracle
import workloads as W

bps = pytest.importorskip("banded_pde_solvers_amd")

LIVE, VREG, EVEN = 1 << 12, 1 << 13, 1 << 14
TRUNK0, SINK = 16, 32


def _lib_or_skip():
    try:
        bps.load_library()
    except bps.BpsLibraryMissing:
        pytest.skip("libbps.so not built")


def _replay(p, u, l, d, rhs, node, code):
    """The two-lane kernel's arithmetic on the host, step by step: slot id s
    of lane j is slots[j][s]; a parent slot flagged EVEN is lane 0's."""
    n = len(p)
    rows = node.shape[1]
    slots = np.zeros((2, SINK + 1, 2))

    def at(j, sid):
        return slots[j], sid

    q = np.full(n, np.nan)
    m = np.full(n, np.nan)
    for t in range(rows):
        rd = []
        for j in (0, 1):                          # read, then clear, the own slot
            c = int(code[j, t])
            arr, sid = at(j, c & 63)
            rd.append(arr[sid].copy())
        for j in (0, 1):
            arr, sid = at(j, int(code[j, t]) & 63)
            arr[sid] = 0.0
        adds = []
        for j in (0, 1):
            c = int(code[j, t])
            x = int(node[j, t])
            dd = (d[x] if x >= 0 else 0.0) - rd[j][0]
            rr = (rhs[x] if x >= 0 else 0.0) - rd[j][1]
            with np.errstate(divide="ignore", invalid="ignore"):
                fac = (u[x] if x >= 0 else 0.0) / dd
            if c & LIVE:
                q[x] = rr / dd
                m[x] = l[x] / dd
            adds.append((at(0 if c & EVEN else j, (c >> 6) & 63), fac * (l[x] if x >= 0 else 0.0),
                         fac * rr))
        for (arr, sid), a0, a1 in adds:
            arr[sid, 0] += a0
            arr[sid, 1] += a1
    V = np.full(n, np.nan)
    slots[:, SINK] = 0.0
    vprev = [0.0, 0.0]
    for t in range(rows - 1, -1, -1):
        vals = []
        for j in (0, 1):
            c = int(code[j, t])
            x = int(node[j, t])
            arr, sid = at(0 if c & EVEN else j, (c >> 6) & 63)
            vp = vprev[j] if c & VREG else arr[sid, 0]
            v = (q[x] - m[x] * vp) if x >= 0 else np.nan
            vals.append((j, c, x, v))
        for j, c, x, v in vals:
            arr, sid = at(j, c & 63)
            arr[sid, 0] = v
            if c & LIVE:
                V[x] = v
                vprev[j] = v
    return V


def _trees():
    rng = np.random.default_rng(77)
    out = []
    for n in (32, 33, 64, 100, 257, 512, 1024, 2048):
        out.append(("window8", W.random_tree(n, rng)))
    for n in (64, 300, 1000):
        out.append(("window16", W.random_tree(n, rng, window=16)))
    # a long trunk with one leaf on every node (a caterpillar) and a comb of
    # long branches: many branch roots on consecutive trunk nodes
    cat = [-1] + [i - 2 if i % 2 == 0 else i - 1 for i in range(1, 401)]
    out.append(("caterpillar", np.array(cat, dtype=np.int32)))
    comb = [-1]
    for i in range(1, 600):
        comb.append(i - 16 if i % 16 == 0 and i >= 16 else i - 1)
    out.append(("comb16", np.array(comb, dtype=np.int32)))
    star = [-1] + [max(0, i - 16) for i in range(1, 200)]
    out.append(("far16", np.array(star, dtype=np.int32)))
    return out


@pytest.mark.parametrize("name,p", _trees(), ids=lambda v: v if isinstance(v, str) else "")
def test_split_schedule_replay_matches_oracle(name, p):
    _lib_or_skip()
    n = len(p)
    sched = bps.hines_split_schedule(p)
    if sched is None:
        pytest.skip(f"{name}: tree stays on one lane")
    node, code = sched
    live = (code & LIVE) != 0
    # every compartment exactly once, the root last on lane 0 in a trunk slot
    assert np.array_equal(np.sort(node[live]), np.arange(n))
    assert np.all(node[~live] == -1)
    assert np.all(code[~live] == SINK | (SINK << 6))
    r0 = np.argwhere(node == 0)
    assert len(r0) == 1 and r0[0][0] == 0 and TRUNK0 <= (code[0, r0[0][1]] & 63) < SINK
    assert r0[0][1] == node.shape[1] - 1 and (code[0, r0[0][1]] >> 6) & 63 == SINK
    assert 5 * node.shape[1] <= 4 * n           # the chain got shorter
    rng = np.random.default_rng(n)
    u = rng.uniform(-1.0, 0.0, n)
    l = rng.uniform(-1.0, 0.0, n)
    u[0] = l[0] = 0.0
    d = 1.0 + np.abs(l) + rng.uniform(0.0, 1.0, n)
    for i in range(1, n):
        d[p[i]] += abs(u[i])
    rhs = rng.uniform(-1.0, 1.0, n)
    V = _replay(p, u, l, d, rhs, node, code)
    ref, info = oracle.hines_solve(p, u, l, d, rhs)
    assert info[0] == 0
    err = np.linalg.norm(V - ref[0]) / np.linalg.norm(ref[0])
    assert err <= 1e-13, (name, err)


def test_split_rows_about_half():
    """On the workloads' trees two lanes take about half the rows of one."""
    _lib_or_skip()
    rng = np.random.default_rng(5)
    for n in (512, 1024, 2048):
        ratios = []
        for _ in range(5):
            s = bps.hines_split_schedule(W.random_tree(n, rng))
            assert s is not None
            ratios.append(s[0].shape[1] / n)
        assert max(ratios) < 0.56, (n, ratios)


def test_split_schedule_arguments():
    _lib_or_skip()
    assert bps.hines_split_schedule(np.array([-1], dtype=np.int32)) is None
    # a chain (all trunk) gains nothing from a second lane
    assert bps.hines_split_schedule(np.r_[-1, np.arange(699)].astype(np.int32)) is None
    # output arrays too short for the schedule: -1 and a message, nothing written past cap
    import ctypes
    L = bps.load_library()
    p = W.random_tree(200, np.random.default_rng(2))
    node = np.full(2 * 10 + 4, -5, dtype=np.int32)
    code = np.zeros(2 * 10 + 4, dtype=np.uint16)
    i32p = ctypes.POINTER(ctypes.c_int32)
    m = L.hines_split_schedule(200, p.ctypes.data_as(i32p), node.ctypes.data_as(i32p),
                               code.ctypes.data_as(ctypes.c_void_p), 10)
    assert m == -1 and "cap" in bps.bps_last_error()
    assert np.all(node == -5)
    with pytest.raises(bps.BpsError):
        bps.hines_split_schedule(np.array([-1, 0, 5], dtype=np.int32))
