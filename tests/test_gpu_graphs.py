"""HIP graphs and concurrent streams, through the C-ABI.

Every solve entry point only enqueues kernels on the given stream (no
allocation, copy, memset or synchronisation), so a sequence of calls can be
captured into a HIP graph and replayed -- the way to amortise launches for
small, launch-bound batches.  Each replay is checked bit for bit against the
eager result, with eager work and synchronisation between replays.  Calls on
two streams with separate buffers give the results of sequential calls."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import banded_pde_solvers_amd as bps
import workloads as W
from gpu_util import buf, dev, host

pytestmark = pytest.mark.gpu


class _Problems:
    """Static device buffers for one call of each kind of solve."""

    def __init__(self):
        rng = np.random.default_rng(3)
        self.C0 = dev(rng.uniform(-1, 1, (1024, 40)))                  # resident hyperdiffusion
        self.C = self.C0.clone()
        self.wh = buf(bps.hyperdiffusion_work_bytes(1024, 40))
        self.Q0 = dev(rng.uniform(-1, 1, (96, 30)))                    # Crank-Nicolson, streaming
        self.Q = self.Q0.clone()
        self.wq = buf(bps.hyperdiffusion_theta_work_bytes(96, 30))
        tb = W.tri_dominant(2048, 50, rng=rng)                         # partitioned tridiagonal
        self.ta, self.tb, self.tc = (dev(v) for v in (tb.a, tb.b, tb.c))
        self.y0 = dev(tb.y)
        self.y = self.y0.clone()
        self.wt = buf(bps.tri_work_bytes(2048, 50))
        hm = W.hines_mono(512, 64, rng=rng)                            # Hines, level schedule
        self.plan = bps.hines_plan_create(64, [512], hm.parent, mono=True,
                                          schedule=bps.BPS_HINES_LEVELS)
        assert self.plan.uses_levels
        self.hu, self.hl, self.hd = (dev(v) for v in (hm.u, hm.l, hm.d))
        self.r0 = dev(hm.rhs)
        self.r = self.r0.clone()
        self.wr = buf(bps.hines_work_bytes(self.plan))
        hs = W.hines_mono(300, 40, rng=rng)                            # Hines, sixteen lanes
        self.splan = bps.hines_plan_create(40, [300], hs.parent, mono=True)
        assert self.splan.uses_sep
        self.su, self.sl, self.sd = (dev(v) for v in (hs.u, hs.l, hs.d))
        self.s0 = dev(hs.rhs)
        self.s = self.s0.clone()
        self.ws = buf(bps.hines_work_bytes(self.splan))
        mm = W.hines_multi(40, 200, 900, rng=rng)                      # multi-morphology, separators
        self.mplan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False)
        assert self.mplan.uses_sep
        mp = []
        for v in (mm.u, mm.l, mm.d, mm.rhs):
            t = torch.empty(self.mplan.elems, dtype=torch.float64, device="cuda:0")
            bps.hines_pack(self.mplan, dev(v), t)
            mp.append(t)
        self.mu, self.ml, self.md, self.m0 = mp
        self.m = self.m0.clone()
        self.wm = buf(bps.hines_work_bytes(self.mplan))
        pb = W.penta_dominant(256, 70, cyclic=True, rng=rng)           # periodic fused penta
        self.pd = [dev(v) for v in pb.diagonals]
        self.x0 = dev(pb.f)
        self.x = self.x0.clone()
        self.wp = buf(bps.bps_penta_work_bytes(256, 70, 70, cyclic=True))

    def reset(self):
        for dst, src in ((self.C, self.C0), (self.Q, self.Q0), (self.y, self.y0),
                         (self.r, self.r0), (self.x, self.x0), (self.s, self.s0), (self.m, self.m0)):
            dst.copy_(src)

    def run(self):
        bps.hyperdiffusion_step(self.C, 1e-6, 1 / 1024, 10, self.wh)
        bps.hyperdiffusion_theta_step(self.Q, 1e-6, 1 / 96, 0.5, 5, self.wq)
        bps.tri_solve_batch(self.ta, self.tb, self.tc, self.y, self.wt)
        bps.hines_solve_batch(self.plan, self.hu, self.hl, self.hd, self.r, self.wr)
        bps.penta_factor_solve_batch(*self.pd, self.x, self.wp, cyclic=True)
        bps.hines_solve_batch(self.splan, self.su, self.sl, self.sd, self.s, self.ws)
        bps.hines_solve_batch(self.mplan, self.mu, self.ml, self.md, self.m, self.wm)

    def outputs(self):
        return [host(t) for t in (self.C, self.Q, self.y, self.r, self.x, self.s, self.m)]


def test_graph_capture_replay_bitwise():
    P = _Problems()
    P.reset()
    P.run()                          # eager: loads every kernel before capture
    torch.cuda.synchronize()
    ref = P.outputs()
    g = torch.cuda.CUDAGraph()
    P.reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        P.run()
    other = W.tri_dominant(512, 20, rng=np.random.default_rng(9))
    for rep in range(3):
        P.reset()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(P.outputs(), ref):
            np.testing.assert_array_equal(got, want)
        # unrelated eager work between replays
        y = dev(other.y)
        bps.tri_solve_batch(dev(other.a), dev(other.b), dev(other.c), y, buf(bps.tri_work_bytes(512, 20)))
        torch.cuda.synchronize()


def test_two_streams_match_sequential():
    A, B = _Problems(), _Problems()
    A.reset(); A.run()
    torch.cuda.synchronize()
    ref = A.outputs()
    A.reset(); B.reset()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        A.run()
    with torch.cuda.stream(s2):
        B.run()
    torch.cuda.synchronize()
    for got_a, got_b, want in zip(A.outputs(), B.outputs(), ref):
        np.testing.assert_array_equal(got_a, want)
        np.testing.assert_array_equal(got_b, want)


def test_first_call_inside_capture():
    """The first library call of a process may be captured: the kernel
    attributes it sets on the device are host-side (tests/graph_first_call.py,
    run as a child process so that nothing before it has touched the
    library)."""
    script = os.path.join(os.path.dirname(os.path.abspath(__file__)), "graph_first_call.py")
    r = subprocess.run([sys.executable, "-u", script], capture_output=True, text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    assert "FIRST_CALL_CAPTURE_OK" in r.stdout
