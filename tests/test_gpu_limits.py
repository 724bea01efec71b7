"""GPU parity at the size limits of each entry point and at degenerate sizes,
against the oracle, through the C-ABI: a tridiagonal system of 16 * 65535
rows (the deepest partitioned path: 65535 chunks, whose interface system is
itself solved one lane per system) and of 2^20 rows (one lane per system),
pentadiagonal systems of 100000 rows (periodic and not), periodic
hyperdiffusion / theta / Cahn-Hilliard on 100000 points (streaming path) and
on n = 6, and a Hines tree of 200000 compartments."""
import numpy as np
import pytest
import torch

import banded_pde_solvers_amd as bps
import oracle
import workloads as W
from gpu_util import TOL, buf, dev, host, info_buf, relerr_cols

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,batch", [(16 * 65535, 3), (1 << 20, 2)])
def test_tridiagonal_longest(n, batch):
    print(f"tri n={n} batch={batch}", flush=True)
    tb = W.tri_dominant(n, batch, rng=np.random.default_rng(1))
    a, b, c, y = (dev(v) for v in (tb.a, tb.b, tb.c, tb.y))
    work = buf(bps.tri_work_bytes(n, batch))
    info = info_buf(batch)
    bps.tri_solve_batch(a, b, c, y, work, info)
    ref, rinfo = oracle.thomas_solve(*(W.to_flat(v) for v in (tb.a, tb.b, tb.c, tb.y)))
    assert relerr_cols(host(y), W.to_interleaved(ref)) <= TOL[torch.float64]
    assert np.all(host(info) == 0) and np.all(rinfo == 0)


@pytest.mark.parametrize("cyclic", [False, True])
def test_pentadiagonal_long(cyclic):
    n, batch = 100000, 3
    print(f"penta n={n} cyclic={cyclic}", flush=True)
    pb = W.penta_dominant(n, batch, cyclic=cyclic, rng=np.random.default_rng(2))
    x = dev(pb.f)
    work = buf(bps.bps_penta_work_bytes(n, batch, batch, cyclic=cyclic))
    info = info_buf(batch)
    bps.penta_factor_solve_batch(*(dev(v) for v in pb.diagonals), x, work, info, cyclic=cyclic)
    ref, rinfo = oracle.penta_solve(*(W.to_flat(v) for v in (*pb.diagonals, pb.f)), cyclic=cyclic)
    assert relerr_cols(host(x), W.to_interleaved(ref)) <= TOL[torch.float64]
    np.testing.assert_array_equal(host(info).astype(int), rinfo)


@pytest.mark.parametrize("n", [100000, 6])
def test_periodic_steps_long_and_shortest(n):
    """Implicit, Crank-Nicolson and Cahn-Hilliard steps; dx = 1/n with a dt
    that keeps sigma moderate (the parity bound then stays 1e-10)."""
    batch = 3
    rng = np.random.default_rng(n)
    C0 = rng.uniform(-1, 1, (n, batch))
    dx = 1.0 / n
    dt = 10.0 * dx ** 4
    C = dev(C0)
    work = buf(bps.hyperdiffusion_work_bytes(n, batch))
    bps.hyperdiffusion_step(C, dt, dx, 3, work)
    ref = oracle.hyperdiffusion(W.to_flat(C0), dt, dx, 3).T
    assert relerr_cols(host(C), ref) <= TOL[torch.float64]
    C = dev(C0)
    work = buf(bps.hyperdiffusion_theta_work_bytes(n, batch))
    bps.hyperdiffusion_theta_step(C, dt, dx, 0.5, 3, work)
    ref = oracle.hyperdiffusion_theta(W.to_flat(C0), dt, dx, 0.5, 3).T
    assert relerr_cols(host(C), ref) <= TOL[torch.float64]
    # Cahn-Hilliard with r = D dt / dx^2 = 0.1 and sigma = gamma r / dx^2 = 10
    C = dev(C0)
    work = buf(bps.cahn_hilliard_work_bytes(n, batch))
    dtc, gamma = 0.1 * dx ** 2, 100.0 * dx ** 2
    bps.cahn_hilliard_step(C, dtc, dx, gamma, 1.0, 1.0, 2, work)
    ref = oracle.cahn_hilliard(W.to_flat(C0), dtc, dx, gamma, 1.0, 1.0, 2).T
    assert relerr_cols(host(C), ref) <= TOL[torch.float64]


def test_hines_large_tree():
    n, batch = 200000, 2
    print(f"hines n={n}", flush=True)
    hm = W.hines_mono(n, batch, rng=np.random.default_rng(3))
    plan = bps.hines_plan_create(batch, [n], hm.parent, mono=True)
    assert not plan.uses_levels
    r = dev(hm.rhs)
    work = buf(bps.hines_work_bytes(plan))
    info = info_buf(batch)
    bps.hines_solve_batch(plan, dev(hm.u), dev(hm.l), dev(hm.d), r, work, info)
    plan.close()
    V, rinfo = oracle.hines_solve(hm.parent, *(W.to_flat(v) for v in (hm.u, hm.l, hm.d, hm.rhs)))
    assert relerr_cols(host(r), W.to_interleaved(V)) <= TOL[torch.float64]
    assert np.all(host(info) == 0) and np.all(rinfo == 0)
