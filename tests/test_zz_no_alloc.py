"""GPU: the allocation-free entry point hyperdiffusion_step_noalloc against
hyperdiffusion_step, through the C-ABI.

Both run the same kernels on the same arithmetic; only the work memory
differs (the library's per-GPU scratch array instead of a caller's buffer),
so the results must be equal bit for bit.  Each case makes two calls in a
row on the shared array, the second with a smaller input (and another path
through the library), so that the second call runs over what the first left
in the array.  Sizes beyond the array are rejected before any launch."""
import numpy as np
import pytest
import torch

import banded_pde_solvers_amd as bps
from gpu_util import buf, dev, host

pytestmark = pytest.mark.gpu


def _reference(C0, dt, dx, nsteps, diagonals=None):
    n, batch = C0.shape
    C = C0.clone()
    code = bps.BPS_F64 if C0.dtype == torch.float64 else bps.BPS_F32
    work = buf(bps.hyperdiffusion_work_bytes(n, batch, code))
    bps.hyperdiffusion_step(C, dt, dx, nsteps, work, diagonals)
    return host(C)


def _noalloc(C0, dt, dx, nsteps, diagonals=None):
    C = C0.clone()
    bps.hyperdiffusion_step_noalloc(C, dt, dx, nsteps, diagonals)
    return host(C)


# (n, batch, dtype, explicit diagonals): resident fp64 path, periodic
# factor + streaming solve (fp32, other n, explicit diagonals)
CASES = [
    ((4096, 40, torch.float64, False), (1024, 300, torch.float64, False)),
    ((18688, 8, torch.float64, False), (256, 64, torch.float64, False)),
    ((2048, 70, torch.float64, False), (96, 33, torch.float32, False)),
    ((37440, 4, torch.float32, False), (512, 50, torch.float64, True)),
    ((1000, 20, torch.float64, True), (100, 9, torch.float32, True)),
]


def _input(n, batch, dtype, explicit, seed):
    rng = np.random.default_rng(seed)
    C0 = dev(rng.uniform(-1, 1, (n, batch)), dtype)
    dg = None
    if explicit:
        # a periodic, symmetric, diagonally dominant operator
        s = rng.uniform(0.5, 2.0)
        v = np.concatenate([np.full(n, s), np.full(n, -4 * s), np.full(n, 1 + 6 * s + 0.5),
                            np.full(n, -4 * s), np.full(n, s)])
        dg = dev(v, dtype)
    return C0, dg


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_step(first, second):
    for k, (n, batch, dtype, explicit) in enumerate((first, second)):
        print(f"noalloc call {k}: n={n} batch={batch} {dtype} explicit={explicit}", flush=True)
        C0, dg = _input(n, batch, dtype, explicit, seed=n + batch + k)
        dt, dx = 1e-6, 1.0 / n
        nsteps = 3 if n > 4096 else 7
        got = _noalloc(C0, dt, dx, nsteps, dg)
        want = _reference(C0, dt, dx, nsteps, dg)
        np.testing.assert_array_equal(got, want)


def test_noalloc_repeated_and_ld():
    """The same call three times, and a leading dimension above the batch
    (padding columns untouched)."""
    n, batch, ld = 1024, 50, 64
    C0 = dev(np.random.default_rng(3).uniform(-1, 1, (n, ld)))
    want = C0.clone()
    bps.hyperdiffusion_step(want, 1e-6, 1.0 / n, 10, buf(bps.hyperdiffusion_work_bytes(n, batch)),
                            batch=batch)
    for _ in range(3):
        C = C0.clone()
        bps.hyperdiffusion_step_noalloc(C, 1e-6, 1.0 / n, 10, batch=batch)
        np.testing.assert_array_equal(host(C), host(want))


def test_noalloc_rejects_sizes_beyond_the_array():
    for n, dtype in ((18726, torch.float64), (37451, torch.float32)):
        C = torch.zeros((n, 2), dtype=dtype, device="cuda:0")
        with pytest.raises(bps.BpsError) as ei:
            bps.hyperdiffusion_step_noalloc(C, 1e-6, 1.0 / n, 1)
        assert ei.value.status == 1
        assert "scratch" in bps.bps_last_error()
    # the largest sizes that fit are accepted
    for n, dtype in ((18725, torch.float64), (37450, torch.float32)):
        code = bps.BPS_F64 if dtype == torch.float64 else bps.BPS_F32
        assert bps.hyperdiffusion_work_bytes(n, 1, code) <= bps.BPS_NOALLOC_SCRATCH_BYTES


def test_noalloc_captured_in_a_graph():
    """The entry point's purpose: a call inside a HIP graph capture (nothing
    allocated while capturing), replayed three times with other work on the
    shared array in between, each replay bitwise equal to an eager call."""
    n, batch = 1024, 64
    rng = np.random.default_rng(21)
    C0 = dev(rng.uniform(-1, 1, (n, batch)))
    C = C0.clone()
    eager = C0.clone()
    bps.hyperdiffusion_step_noalloc(eager, 1e-6, 1.0 / n, 5)
    want = host(eager)
    other = dev(rng.uniform(-1, 1, (96, 10)))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bps.hyperdiffusion_step_noalloc(C, 1e-6, 1.0 / n, 5)
    for _ in range(3):
        C.copy_(C0)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(C), want)
        # another size through the same scratch array between replays
        bps.hyperdiffusion_step_noalloc(other, 1e-6, 1.0 / 96, 2)
        torch.cuda.synchronize()
