"""GPU parity: semi-implicit periodic Cahn-Hilliard steps (cahn_hilliard_step)
against the oracle, through the C-ABI.

Tolerance.  The explicit side adds r D2 (C^3 - C) to the theta-scheme
stencil; its rounding is at most ~u (1 + 16 (1-theta) sigma + 16 r) |C| per
row, and the implicit solve then has the forward error of the theta-scheme
step (order kappa u with kappa = 1 + 16 theta sigma when theta < 1 keeps the
high modes at O(1)).  Each one-step comparison therefore allows
max(base, 4 u (kappa + 16 r)), base = 1e-10 (fp64) or 1e-4 (fp32 against the
fp64 oracle of the fp32-rounded state).  Over k steps the difference between
two trajectories grows at most by the Lipschitz constant L of one step of the
linearised scheme (max over modes of (|mu_k| + r m_k max|3C^2 - 1|) / lambda_k,
computed from the operators), so a k-step trajectory allows
tol * (1 + L + ... + L^(k-1)) relative to ||C0||.  A wrong sign, index or
coefficient gives errors of the size of the phase-separation term itself,
orders of magnitude above these bounds."""
import numpy as np
import pytest
import torch

import banded_pde_solvers_amd as bps
import oracle
import workloads as W
from gpu_util import TOL, buf, dev, host, relerr_cols, rounded

pytestmark = pytest.mark.gpu

GAMMA, MOB = 1e-4, 1.0


def _tol(n, dt, dx, gamma, mob, theta, dtype=torch.float64):
    u = float(np.finfo(np.float64 if dtype == torch.float64 else np.float32).eps) / 2
    r = mob * dt / dx ** 2
    sigma = gamma * r / dx ** 2
    kappa = 1 + 16 * theta * sigma
    return max(TOL[dtype], 4 * u * (kappa + 16 * r))


def _lipschitz(n, dt, dx, gamma, mob, theta, cmax):
    (e2, e1, e0), r, dg = oracle.cahn_hilliard_operators(n, dt, dx, gamma, mob, theta)
    th = 2 * np.pi * np.arange(n) / n
    lam = dg[2][0] + 2 * dg[1][0] * np.cos(th) + 2 * dg[0][0] * np.cos(2 * th)
    mu = e0 + 2 * e1 * np.cos(th) + 2 * e2 * np.cos(2 * th)
    m = 2 - 2 * np.cos(th)
    lphi = max(1.0, 3 * cmax ** 2 - 1)
    return float(np.max((np.abs(mu) + r * m * lphi) / lam))


def _traj_tol(n, dt, dx, gamma, mob, theta, k, cmax=1.0):
    L = _lipschitz(n, dt, dx, gamma, mob, theta, cmax)
    return _tol(n, dt, dx, gamma, mob, theta) * sum(L ** j for j in range(k))


def _run(C0, dt, dx, theta, nsteps, dtype=torch.float64, gamma=GAMMA, mob=MOB, batch=None):
    n = C0.shape[0]
    C = dev(C0, dtype)
    b = C0.shape[1] if batch is None else batch
    code = bps.BPS_F64 if dtype == torch.float64 else bps.BPS_F32
    work = buf(bps.cahn_hilliard_work_bytes(n, b, code))
    bps.cahn_hilliard_step(C, dt, dx, gamma, mob, theta, nsteps, work, batch=batch)
    return host(C)


def _oracle(C0, dt, dx, theta, nsteps, dtype=torch.float64, gamma=GAMMA, mob=MOB):
    return oracle.cahn_hilliard(W.to_flat(rounded(C0, dtype)), dt, dx, gamma, mob, theta, nsteps).T


@pytest.mark.parametrize("theta", [1.0, 0.5, 0.3])
@pytest.mark.parametrize("n,batch", [(128, 37), (256, 17), (1024, 100), (832, 20), (2048, 24), (4096, 10), (512, 21), (768, 13),   # resident
                                     (96, 50), (100, 33)])                          # streaming
def test_one_step_parity(n, batch, theta):
    print(f"theta={theta} n={n} batch={batch}", flush=True)
    rng = np.random.default_rng(n + batch + 1)
    C0 = rng.uniform(-1, 1, (n, batch))
    dt, dx = 1e-6, 1.0 / n
    got = _run(C0, dt, dx, theta, 1)
    ref = _oracle(C0, dt, dx, theta, 1)
    assert relerr_cols(got, ref) <= _tol(n, dt, dx, GAMMA, MOB, theta)


@pytest.mark.parametrize("n", [256, 100])
@pytest.mark.parametrize("theta", [1.0, 0.5])
def test_fp32(n, theta):
    rng = np.random.default_rng(17)
    C0 = rng.uniform(-1, 1, (n, 40))
    dt, dx = 1e-6, 1.0 / n
    got = _run(C0, dt, dx, theta, 1, torch.float32)
    ref = _oracle(C0, dt, dx, theta, 1, torch.float32)
    assert relerr_cols(got, ref) <= _tol(n, dt, dx, GAMMA, MOB, theta, torch.float32)


@pytest.mark.parametrize("n,nsteps,theta", [(1024, 20, 1.0), (1024, 20, 0.5), (256, 40, 1.0),
                                            (96, 20, 1.0), (96, 20, 0.5)])
def test_trajectory(n, nsteps, theta):
    rng = np.random.default_rng(n + nsteps)
    C0 = rng.uniform(-1, 1, (n, 33))
    dt, dx = 1e-6, 1.0 / n
    got = _run(C0, dt, dx, theta, nsteps)
    ref = _oracle(C0, dt, dx, theta, nsteps)
    err = np.linalg.norm(got - ref, axis=0) / np.linalg.norm(C0, axis=0)
    cmax = max(1.0, float(np.max(np.abs(ref))))
    assert np.max(err) <= _traj_tol(n, dt, dx, GAMMA, MOB, theta, nsteps, cmax)


def test_steps_compose():
    """k steps in one call equal k calls of one step (resident path), bit for bit."""
    n = 512
    rng = np.random.default_rng(14)
    C0 = rng.uniform(-1, 1, (n, 40))
    dt, dx = 1e-6, 1.0 / n
    for theta in (1.0, 0.5):
        once = _run(C0, dt, dx, theta, 6)
        C = dev(C0)
        work = buf(bps.cahn_hilliard_work_bytes(n, 40))
        for _ in range(6):
            bps.cahn_hilliard_step(C, dt, dx, GAMMA, MOB, theta, 1, work)
        np.testing.assert_array_equal(once, host(C))


@pytest.mark.parametrize("n", [1024, 96])
def test_leading_dimension_and_untouched_columns(n):
    batch, ld = 30, 48
    rng = np.random.default_rng(22)
    C0 = rng.uniform(-1, 1, (n, ld))
    dt, dx = 1e-6, 1.0 / n
    out = _run(C0, dt, dx, 1.0, 3, batch=batch)
    ref = _oracle(C0[:, :batch], dt, dx, 1.0, 3)
    err = np.linalg.norm(out[:, :batch] - ref, axis=0) / np.linalg.norm(C0[:, :batch], axis=0)
    assert np.max(err) <= _traj_tol(n, dt, dx, GAMMA, MOB, 1.0, 3)
    np.testing.assert_array_equal(out[:, batch:], C0[:, batch:])


@pytest.mark.parametrize("n", [1024, 100])
def test_mass_conserved_and_constants_fixed(n):
    """Column sums are preserved over 50 steps; constant columns stay
    constant.  The phase-separation term of a constant is exactly zero, so a
    constant is multiplied by 1 / lambda_0 per step, lambda_0 = c + 2b + 2a
    the constant-mode eigenvalue of the stored fp64 diagonals (1 only up to
    their rounding: ~1e-13 at sigma = 110), up to the solve's own rounding,
    at most ~4 kappa u per step."""
    rng = np.random.default_rng(31)
    C0 = rng.uniform(-0.5, 0.5, (n, 20)) + 0.1
    C0[:, 0] = 0.37
    C0[:, 1] = -1.0
    dt, dx = 1e-6, 1.0 / n
    got = _run(C0, dt, dx, 1.0, 50)
    np.testing.assert_allclose(got.sum(axis=0), C0.sum(axis=0), rtol=0, atol=1e-10 * n)
    _, _, dg = oracle.cahn_hilliard_operators(n, dt, dx, GAMMA, MOB, 1.0)
    lam0 = np.longdouble(dg[2][0]) + 2 * np.longdouble(dg[1][0]) + 2 * np.longdouble(dg[0][0])
    g50 = float(1 / lam0 ** 50)
    u = np.finfo(np.float64).eps / 2
    kappa = float(dg[2][0] - 2 * dg[1][0] + 2 * dg[0][0])     # largest eigenvalue
    for col, c0 in ((0, 0.37), (1, -1.0)):
        np.testing.assert_allclose(got[:, col], c0 * g50, rtol=0, atol=50 * 4 * kappa * u * abs(c0))


def test_spinodal_growth_on_gpu():
    """A long-wave perturbation of the mixed state grows, one of a stable
    state (c0 = 0.8) decays, as the oracle's linearised factor predicts."""
    n = 1024
    dt, dx = 1e-6, 1.0 / n
    x = np.arange(n) / n
    C0 = np.stack([1e-4 * np.cos(2 * np.pi * 4 * x), 0.8 + 1e-4 * np.cos(2 * np.pi * 4 * x)], axis=1)
    got = _run(C0, dt, dx, 1.0, 50)
    amp = np.abs(np.fft.fft(got, axis=0)[4]) / np.abs(np.fft.fft(C0, axis=0)[4])
    assert amp[0] > 1.0 and amp[1] < 1.0, amp


def test_invalid_arguments():
    C = dev(np.zeros((64, 4)))
    work = buf(bps.cahn_hilliard_work_bytes(64, 4))
    for gamma, mob, th in ((-1e-4, 1.0, 1.0), (1e-4, float("nan"), 1.0), (1e-4, 1.0, 1.5),
                           (float("inf"), 1.0, 1.0)):
        with pytest.raises(bps.BpsError):
            bps.cahn_hilliard_step(C, 1e-6, 1.0 / 64, gamma, mob, th, 1, work)


@pytest.mark.slow
def test_cahn_hilliard_full_sampled():
    """N = 1024, 16384 systems, 100 semi-implicit steps in one call, as
    benchmarked: sampled systems against the oracle's trajectory, plus a
    one-step check."""
    cfg = W.WORKLOADS[6]
    n, batch, dt, dx = cfg["n"], cfg["batch"], cfg["dt"], cfg["dx"]
    g, mob, theta, k = cfg["gamma"], cfg["mobility"], cfg["theta"], cfg["nsteps"]
    print(f"full Cahn-Hilliard workload {n}x{batch}", flush=True)
    C0 = W.cahn_hilliard_quench(n, batch)
    out = _run(C0, dt, dx, theta, k, gamma=g, mob=mob)
    cols = np.unique(np.r_[0, 15, 16, batch - 1, np.random.default_rng(6).integers(0, batch, 40)])
    ref = _oracle(C0[:, cols], dt, dx, theta, k, gamma=g, mob=mob)
    err = np.linalg.norm(out[:, cols] - ref, axis=0) / np.linalg.norm(C0[:, cols], axis=0)
    assert np.max(err) <= _traj_tol(n, dt, dx, g, mob, theta, k)
    one = _run(C0, dt, dx, theta, 1, gamma=g, mob=mob)
    ref1 = _oracle(C0[:, cols], dt, dx, theta, 1, gamma=g, mob=mob)
    assert relerr_cols(one[:, cols], ref1) <= _tol(n, dt, dx, g, mob, theta)
