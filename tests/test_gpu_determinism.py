"""Run-to-run bitwise determinism of every solver path, and agreement of
paths that compute the same thing in a different order (through the C-ABI).

The level schedule of the Hines solver adds sibling contributions with LDS
atomics; within one wavefront those are applied in a fixed order, so it is
checked bitwise too."""
import numpy as np
import pytest
import torch

import banded_pde_solvers_amd as bps
import workloads as W
from gpu_util import buf, dev, host, relerr_cols

pytestmark = pytest.mark.gpu


def _twice(fn):
    a = fn()
    b = fn()
    np.testing.assert_array_equal(a, b)
    return a


@pytest.mark.parametrize("n", [512, 2048, 1000])       # chunked, partitioned, one lane
def test_tridiagonal_bitwise(n):
    tb = W.tri_dominant(n, 300, rng=np.random.default_rng(n))

    def run():
        y = dev(tb.y)
        bps.tri_solve_batch(dev(tb.a), dev(tb.b), dev(tb.c), y, buf(bps.tri_work_bytes(n, 300)))
        return host(y)
    _twice(run)


@pytest.mark.parametrize("schedule", [bps.BPS_HINES_LANES, bps.BPS_HINES_LEVELS])
def test_hines_bitwise(schedule):
    hm = W.hines_mono(512, 200, rng=np.random.default_rng(5))
    mm = W.hines_multi(150, 100, 900, rng=np.random.default_rng(6))

    def run_mono():
        plan = bps.hines_plan_create(200, [512], hm.parent, mono=True, schedule=schedule)
        r = dev(hm.rhs)
        bps.hines_solve_batch(plan, dev(hm.u), dev(hm.l), dev(hm.d), r, buf(bps.hines_work_bytes(plan)))
        plan.close()
        return host(r)

    def run_multi():
        plan = bps.hines_plan_create(mm.batch, mm.sizes, mm.parent, mono=False, schedule=schedule)
        pk = [torch.empty(plan.elems, dtype=torch.float64, device="cuda:0") for _ in range(4)]
        for src, dst in zip((mm.u, mm.l, mm.d, mm.rhs), pk):
            bps.hines_pack(plan, dev(src), dst)
        bps.hines_solve_batch(plan, *pk, buf(bps.hines_work_bytes(plan)))
        out = torch.empty(len(mm.u), dtype=torch.float64, device="cuda:0")
        bps.hines_unpack(plan, pk[3], out)
        plan.close()
        return host(out)
    _twice(run_mono)
    _twice(run_multi)


@pytest.mark.parametrize("n", [1024, 96])                 # resident, streaming
def test_theta_and_cahn_hilliard_bitwise(n):
    C0 = np.random.default_rng(n).uniform(-1, 1, (n, 70))
    dx = 1.0 / n

    def theta():
        C = dev(C0)
        bps.hyperdiffusion_theta_step(C, 1e-6, dx, 0.5, 7, buf(bps.hyperdiffusion_theta_work_bytes(n, 70)))
        return host(C)

    def ch():
        C = dev(C0)
        bps.cahn_hilliard_step(C, 1e-6, dx, 1e-4, 1.0, 1.0, 7, buf(bps.cahn_hilliard_work_bytes(n, 70)))
        return host(C)
    _twice(theta)
    _twice(ch)


@pytest.mark.parametrize("n", [256, 96])                  # chunked, second pass only
def test_periodic_fused_bitwise_and_equal_to_split(n):
    batch = 120
    pb = W.penta_dominant(n, batch, cyclic=True, rng=np.random.default_rng(n + 3))

    def fused():
        x = dev(pb.f)
        bps.penta_factor_solve_batch(*(dev(v) for v in pb.diagonals), x,
                                     buf(bps.bps_penta_work_bytes(n, batch, batch, cyclic=True)),
                                     cyclic=True)
        return host(x)
    a = _twice(fused)
    fac = buf(bps.bps_penta_factor_bytes(n, batch, batch, bps.BPS_F64, bps.BPS_CYCLIC))
    bps.penta_factor_batch(*(dev(v) for v in pb.diagonals), fac, cyclic=True)
    x = dev(pb.f)
    bps.penta_cyclic_solve_batch(fac, x)
    assert relerr_cols(a, host(x)) <= 1e-13
