"""GPU parity: theta-scheme periodic hyperdiffusion (hyperdiffusion_theta_step)
against the oracle, through the C-ABI.

Tolerance.  Unlike the fully implicit step, whose output is dominated by the
slowly decaying low modes, a theta < 1 step keeps the high modes at O(1)
(Crank-Nicolson maps them to about -1).  A backward-stable solve with
A = I + theta sigma D4 then has a normwise forward error of order kappa(A) u,
where kappa(A) = 1 + 16 theta sigma is the ratio of the extreme eigenvalues of
that symmetric positive definite circulant (1 for the constant mode,
1 + 16 theta sigma for the alternating one) and u the unit roundoff.  At
n = 1024, dt = 1e-6 this is ~1e-9 in fp64: two correct fp64 solvers (a dense
LAPACK solve and the oracle) already differ by 0.6 kappa u there.  Each
one-step comparison therefore allows max(base, 4 kappa u), base = 1e-10 (fp64)
or 1e-4 (fp32 against the fp64 oracle of the fp32-rounded state); a
trajectory of k steps allows k times that, since for theta >= 1/2 every mode
factor has magnitude <= 1 and per-step errors add at most linearly.  A wrong
term, sign or index gives O(1) errors, far above these bounds.  theta = 1 must
reproduce hyperdiffusion_step bit for bit."""
import numpy as np
import pytest
import torch

import banded_pde_solvers_amd as bps
import oracle
import workloads as W
from gpu_util import TOL, buf, dev, host, relerr_cols, rounded

pytestmark = pytest.mark.gpu


def _tol(n, dt, dx, theta, dtype=torch.float64):
    u = float(np.finfo(np.float64 if dtype == torch.float64 else np.float32).eps) / 2
    kappa = 1 + 16 * theta * dt / dx ** 4
    return max(TOL[dtype], 4 * kappa * u)


def _run(C0, dt, dx, theta, nsteps, dtype=torch.float64):
    n, batch = C0.shape
    C = dev(C0, dtype)
    code = bps.BPS_F64 if dtype == torch.float64 else bps.BPS_F32
    work = buf(bps.hyperdiffusion_theta_work_bytes(n, batch, code))
    bps.hyperdiffusion_theta_step(C, dt, dx, theta, nsteps, work)
    return host(C)


def _oracle(C0, dt, dx, theta, nsteps, dtype=torch.float64):
    return oracle.hyperdiffusion_theta(W.to_flat(rounded(C0, dtype)), dt, dx, theta, nsteps).T


@pytest.mark.parametrize("theta", [0.5, 0.3, 0.75])
@pytest.mark.parametrize("n,batch", [(128, 37), (256, 17), (1024, 100), (832, 20), (2048, 24), (4096, 10),   # resident
                                     (96, 50), (100, 33)])                          # streaming
def test_one_step_parity(n, batch, theta):
    print(f"theta={theta} n={n} batch={batch}", flush=True)
    rng = np.random.default_rng(n + batch)
    C0 = rng.uniform(-1, 1, (n, batch))
    dt, dx = 1e-6, 1.0 / n
    got = _run(C0, dt, dx, theta, 1)
    ref = _oracle(C0, dt, dx, theta, 1)
    assert relerr_cols(got, ref) <= _tol(n, dt, dx, theta)


@pytest.mark.parametrize("n", [256, 100])
def test_fp32(n):
    rng = np.random.default_rng(7)
    C0 = rng.uniform(-1, 1, (n, 40))
    dt, dx = 1e-8, 1.0 / n
    got = _run(C0, dt, dx, 0.5, 1, torch.float32)
    ref = _oracle(C0, dt, dx, 0.5, 1, torch.float32)
    assert relerr_cols(got, ref) <= _tol(n, dt, dx, 0.5, torch.float32)


@pytest.mark.parametrize("n", [1024, 96])
def test_theta_one_equals_implicit_step(n):
    rng = np.random.default_rng(9)
    C0 = rng.uniform(-1, 1, (n, 70))
    dt, dx = 1e-6, 1.0 / n
    a = _run(C0, dt, dx, 1.0, 5)
    C = dev(C0)
    work = buf(bps.hyperdiffusion_work_bytes(n, 70))
    bps.hyperdiffusion_step(C, dt, dx, 5, work)
    np.testing.assert_array_equal(a, host(C))


@pytest.mark.parametrize("n,nsteps", [(1024, 20), (256, 50), (96, 20)])
def test_trajectory(n, nsteps):
    """Crank-Nicolson, several steps in one call."""
    rng = np.random.default_rng(n)
    C0 = rng.uniform(-1, 1, (n, 33))
    dt, dx = 1e-6, 1.0 / n
    got = _run(C0, dt, dx, 0.5, nsteps)
    ref = _oracle(C0, dt, dx, 0.5, nsteps)
    err = np.linalg.norm(got - ref, axis=0) / np.linalg.norm(C0, axis=0)
    assert np.max(err) <= nsteps * _tol(n, dt, dx, 0.5)


def test_steps_compose():
    """k steps in one call equal k calls of one step (resident path), bit for bit."""
    n = 512
    rng = np.random.default_rng(4)
    C0 = rng.uniform(-1, 1, (n, 40))
    dt, dx = 1e-6, 1.0 / n
    once = _run(C0, dt, dx, 0.5, 6)
    C = dev(C0)
    work = buf(bps.hyperdiffusion_theta_work_bytes(n, 40))
    for _ in range(6):
        bps.hyperdiffusion_theta_step(C, dt, dx, 0.5, 1, work)
    np.testing.assert_array_equal(once, host(C))


def test_leading_dimension_and_untouched_columns():
    n, batch, ld = 1024, 30, 48
    rng = np.random.default_rng(12)
    C0 = rng.uniform(-1, 1, (n, ld))
    dt, dx = 1e-6, 1.0 / n
    C = dev(C0)
    work = buf(bps.hyperdiffusion_theta_work_bytes(n, batch))
    bps.hyperdiffusion_theta_step(C, dt, dx, 0.5, 3, work, batch=batch)
    out = host(C)
    ref = _oracle(C0[:, :batch], dt, dx, 0.5, 3)
    err = np.linalg.norm(out[:, :batch] - ref, axis=0) / np.linalg.norm(C0[:, :batch], axis=0)
    assert np.max(err) <= 3 * _tol(n, dt, dx, 0.5)
    np.testing.assert_array_equal(out[:, batch:], C0[:, batch:])


def test_invalid_theta():
    C = dev(np.zeros((64, 4)))
    work = buf(bps.hyperdiffusion_theta_work_bytes(64, 4))
    for th in (-0.1, 1.5, float("nan")):
        with pytest.raises(bps.BpsError):
            bps.hyperdiffusion_theta_step(C, 1e-6, 1.0 / 64, th, 1, work)


@pytest.mark.slow
def test_crank_nicolson_full_sampled():
    """N = 1024, 16384 systems, 100 Crank-Nicolson steps in one call, as
    benchmarked: sampled systems against the oracle's trajectory (per-step
    error bound times the step count), plus a one-step check."""
    cfg = W.WORKLOADS[5]
    n, batch, dt, dx, theta = cfg["n"], cfg["batch"], cfg["dt"], cfg["dx"], cfg["theta"]
    print(f"full Crank-Nicolson workload {n}x{batch}", flush=True)
    C0 = W.hyperdiffusion_random(n, batch)
    out = _run(C0, dt, dx, theta, cfg["nsteps"])
    cols = np.unique(np.r_[0, 15, 16, batch - 1, np.random.default_rng(5).integers(0, batch, 40)])
    ref = _oracle(C0[:, cols], dt, dx, theta, cfg["nsteps"])
    err = np.linalg.norm(out[:, cols] - ref, axis=0) / np.linalg.norm(C0[:, cols], axis=0)
    assert np.max(err) <= cfg["nsteps"] * _tol(n, dt, dx, theta)
    one = _run(C0, dt, dx, theta, 1)
    assert relerr_cols(one[:, cols], _oracle(C0[:, cols], dt, dx, theta, 1)) <= _tol(n, dt, dx, theta)


@pytest.mark.parametrize("n", [1024, 96])
def test_theta_zero_time_step_is_identity(n):
    """dt = 0: both sides of the theta scheme are I."""
    C0 = np.random.default_rng(n + 3).uniform(-1, 1, (n, 24))
    C = dev(C0)
    work = buf(bps.hyperdiffusion_theta_work_bytes(n, 24))
    bps.hyperdiffusion_theta_step(C, 0.0, 1.0 / n, 0.5, 5, work)
    np.testing.assert_allclose(host(C), C0, rtol=0, atol=1e-15)
