"""GPU parity: theta-scheme periodic hyperdiffusion (hyperdiffusion_theta_step)
against the oracle, through the C-ABI, both refereed by the exact solution.

Unlike the fully implicit step, whose output is dominated by the slowly
decaying low modes, a theta < 1 step keeps the high modes at O(1)
(Crank-Nicolson maps them to about -1), so a backward-stable solve with
A = I + theta sigma D4 (kappa = 1 + 16 theta sigma, ~8.8e6 at n = 1024,
dt = 1e-6, theta = 1/2) has a forward error of order kappa u: two correct
fp64 solvers differ by ~1e-10 .. 1e-9 there.  The referee is the exact map
of the stored operator: both matrices are circulant, so one step multiplies
discrete Fourier mode k by mu_k / lambda_k, with mu_k and lambda_k the
symbols of the explicit stencil (-se, 4 se, 1 - 6 se, 4 se, -se) and of the
implicit matrix (si, -4 si, 1 + 6 si, -4 si, si), evaluated from the fp64
entries in extended precision (si = theta sigma, se = (1 - theta) sigma,
sigma = dt / (dx dx dx dx), rounded as the operator is defined).  Each test
measures, per system, the GPU's and the oracle's normwise errors against it
and requires every GPU error to be at most max(1e-10, twice the largest
oracle error of the batch) and the GPU's mean error at most max(1e-10, three
times the oracle's); GPU against oracle is then bounded by the triangle
inequality, max(1e-10, three times that largest oracle error).  The batch's
worst and mean errors are compared, not each system's: the oracle's
per-system error varies tenfold with the right-hand side (at n = 1024,
theta = 1/2: 3.5e-11 .. 3.3e-10), the chunked GPU solve's about twofold,
both at 0.1 .. 0.4 kappa u.  A wrong term, sign or index gives O(1) errors;
a systematic defect of 1e-9 per step fails the mean check at n = 1024.
theta = 1 must reproduce hyperdiffusion_step bit for bit."""
import numpy as np
import pytest
import torch

import banded_pde_solvers_amd as bps
import oracle
import workloads as W
from gpu_util import TOL, buf, dev, host, relerr_cols, rounded

pytestmark = pytest.mark.gpu


def _tol(n, dt, dx, theta, dtype=torch.float64):
    """fp32 only: the fp64 oracle of the fp32-rounded state, base 1e-4 (the
    kappa u of fp32 stays below it at the tested sizes)."""
    u = float(np.finfo(np.float64 if dtype == torch.float64 else np.float32).eps) / 2
    kappa = 1 + 16 * theta * dt / dx ** 4
    return max(TOL[dtype], 4 * kappa * u)


def _exact(C0, dt, dx, theta, nsteps):
    """The exact theta steps of the stored fp64 operator on interleaved C0
    (n, batch): mode k times (mu_k / lambda_k)^nsteps, symbols in extended
    precision, one fp64 FFT pair."""
    n = C0.shape[0]
    sigma = dt / (dx * dx * dx * dx)
    si, se = theta * sigma, (1.0 - theta) * sigma
    a, b, c = si, -4.0 * si, 1.0 + 6.0 * si
    e2, e1, e0 = -se, 4.0 * se, 1.0 - 6.0 * se
    L = np.longdouble
    th = 2 * np.pi * np.arange(n, dtype=L) / n
    lam = L(c) + 2 * L(b) * np.cos(th) + 2 * L(a) * np.cos(2 * th)
    mu = L(e0) + 2 * L(e1) * np.cos(th) + 2 * L(e2) * np.cos(2 * th)
    g = ((mu / lam) ** nsteps).astype(float)
    return np.real(np.fft.ifft(np.fft.fft(C0, axis=0) * g[:, None], axis=0))


def _referee(got, ref, ex, scale, what):
    """Per-system errors of the GPU (got) and the oracle (ref) against the
    exact solution (ex), relative to the norms in `scale` (n, batch);
    asserts the bounds of the module docstring and returns the largest
    oracle error."""
    den = np.linalg.norm(scale, axis=0)
    e_gpu = np.linalg.norm(got - ex, axis=0) / den
    e_orc = np.linalg.norm(ref - ex, axis=0) / den
    print(f"{what}: GPU vs exact max {e_gpu.max():.3e} mean {e_gpu.mean():.3e}; "
          f"oracle vs exact max {e_orc.max():.3e} mean {e_orc.mean():.3e}", flush=True)
    bound = max(1e-10, 2 * float(e_orc.max()))
    assert np.all(e_gpu <= bound), (e_gpu.max(), bound)
    assert e_gpu.mean() <= max(1e-10, 3 * e_orc.mean()), (e_gpu.mean(), e_orc.mean())
    return float(e_orc.max())


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
@pytest.mark.parametrize("n,batch", [(128, 37), (256, 17), (1024, 100), (832, 20), (2048, 24), (4096, 10), (512, 21), (768, 13),   # resident
                                     (96, 50), (100, 33)])                          # streaming
def test_one_step_parity(n, batch, theta):
    print(f"theta={theta} n={n} batch={batch}", flush=True)
    rng = np.random.default_rng(n + batch)
    C0 = rng.uniform(-1, 1, (n, batch))
    dt, dx = 1e-6, 1.0 / n
    got = _run(C0, dt, dx, theta, 1)
    ref = _oracle(C0, dt, dx, theta, 1)
    ex = _exact(C0, dt, dx, theta, 1)
    e_orc = _referee(got, ref, ex, ex, f"one step n={n} theta={theta}")
    assert relerr_cols(got, ref) <= max(1e-10, 3 * e_orc)


@pytest.mark.parametrize("theta", [0.5, 0.75])
def test_referee_workload_shape(theta):
    """N = 1024 (the Crank-Nicolson workload's grid), 256 systems: one step
    against the exact circulant solution, GPU and oracle alike."""
    n, batch = 1024, 256
    rng = np.random.default_rng(31)
    C0 = rng.uniform(-1, 1, (n, batch))
    dt, dx = 1e-6, 1.0 / n
    got = _run(C0, dt, dx, theta, 1)
    ref = _oracle(C0, dt, dx, theta, 1)
    ex = _exact(C0, dt, dx, theta, 1)
    e_orc = _referee(got, ref, ex, ex, f"referee n=1024 theta={theta}")
    assert relerr_cols(got, ref) <= max(1e-10, 3 * e_orc)


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
    """Crank-Nicolson, several steps in one call: the trajectory against the
    exact one (errors relative to the norm of C0), GPU and oracle alike."""
    rng = np.random.default_rng(n)
    C0 = rng.uniform(-1, 1, (n, 33))
    dt, dx = 1e-6, 1.0 / n
    got = _run(C0, dt, dx, 0.5, nsteps)
    ref = _oracle(C0, dt, dx, 0.5, nsteps)
    ex = _exact(C0, dt, dx, 0.5, nsteps)
    e_orc = _referee(got, ref, ex, C0, f"{nsteps}-step trajectory n={n}")
    err = np.linalg.norm(got - ref, axis=0) / np.linalg.norm(C0, axis=0)
    assert np.max(err) <= max(1e-10, 3 * e_orc)


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
    ex = _exact(C0[:, :batch], dt, dx, 0.5, 3)
    e_orc = _referee(out[:, :batch], ref, ex, C0[:, :batch], "ld 48, 30 systems, 3 steps")
    err = np.linalg.norm(out[:, :batch] - ref, axis=0) / np.linalg.norm(C0[:, :batch], axis=0)
    assert np.max(err) <= max(1e-10, 3 * e_orc)
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
    benchmarked: sampled systems against the exact trajectory, GPU and oracle
    alike, plus a one-step check."""
    cfg = W.WORKLOADS[5]
    n, batch, dt, dx, theta = cfg["n"], cfg["batch"], cfg["dt"], cfg["dx"], cfg["theta"]
    print(f"full Crank-Nicolson workload {n}x{batch}", flush=True)
    C0 = W.hyperdiffusion_random(n, batch)
    out = _run(C0, dt, dx, theta, cfg["nsteps"])
    cols = np.unique(np.r_[0, 15, 16, batch - 1, np.random.default_rng(5).integers(0, batch, 40)])
    ref = _oracle(C0[:, cols], dt, dx, theta, cfg["nsteps"])
    ex = _exact(C0[:, cols], dt, dx, theta, cfg["nsteps"])
    e_orc = _referee(out[:, cols], ref, ex, C0[:, cols], "full workload, 100 steps")
    err = np.linalg.norm(out[:, cols] - ref, axis=0) / np.linalg.norm(C0[:, cols], axis=0)
    assert np.max(err) <= max(1e-10, 3 * e_orc)
    one = _run(C0, dt, dx, theta, 1)
    ex1 = _exact(C0[:, cols], dt, dx, theta, 1)
    ref1 = _oracle(C0[:, cols], dt, dx, theta, 1)
    e1 = _referee(one[:, cols], ref1, ex1, ex1, "full workload, one step")
    assert relerr_cols(one[:, cols], ref1) <= max(1e-10, 3 * e1)


@pytest.mark.parametrize("n", [1024, 96])
def test_theta_zero_time_step_is_identity(n):
    """dt = 0: both sides of the theta scheme are I."""
    C0 = np.random.default_rng(n + 3).uniform(-1, 1, (n, 24))
    C = dev(C0)
    work = buf(bps.hyperdiffusion_theta_work_bytes(n, 24))
    bps.hyperdiffusion_theta_step(C, 0.0, 1.0 / n, 0.5, 5, work)
    np.testing.assert_allclose(host(C), C0, rtol=0, atol=1e-15)
