"""Pins for the oracle's theta-scheme hyperdiffusion step (cuPentBatch page,
hyperdiffusion section: the page time-steps with Crank-Nicolson, theta = 1/2):

    (I + theta sigma D4) C^{k+1} = (I - (1 - theta) sigma D4) C^k,  sigma = dt/dx^4.

Independent checks: dense LAPACK solves of the same periodic matrices on
small grids, the exact per-step factor of a single Fourier mode (eigenvalues
of both circulant operators from the stored fp64 entries, in extended
precision), theta = 1 reproducing the implicit step, mean conservation, and
the temporal convergence order of the scheme against the semi-discrete
exact decay (order 2 for Crank-Nicolson, order 1 for backward Euler)."""
import math

import numpy as np
import pytest

import oracle
from dense import cyclic_dense, relerr


def _stencil_dense(n, e2, e1, e0):
    B = np.zeros((n, n))
    for i in range(n):
        for off, v in ((-2, e2), (-1, e1), (0, e0), (1, e1), (2, e2)):
            B[i, (i + off) % n] += v
    return B


@pytest.mark.parametrize("n", [6, 7, 9, 16])
@pytest.mark.parametrize("theta", [0.0, 0.3, 0.5, 1.0])
def test_matches_dense_lapack(n, theta):
    rng = np.random.default_rng(n * 10 + int(theta * 10))
    dt, dx = 0.02, 1.0 / n
    (e2, e1, e0), dg = oracle.hyperdiffusion_theta_operators(n, dt, dx, theta)
    A = cyclic_dense(*dg)
    B = _stencil_dense(n, e2, e1, e0)
    C0 = rng.uniform(-1, 1, (3, n))
    got = oracle.hyperdiffusion_theta(C0, dt, dx, theta, 3)
    ref = C0.T.copy()
    for _ in range(3):
        ref = np.linalg.solve(A, B @ ref)
    assert relerr(got, ref.T) < 1e-12


def test_theta_one_is_the_implicit_step():
    rng = np.random.default_rng(3)
    C0 = rng.uniform(-1, 1, (5, 256))
    a = oracle.hyperdiffusion_theta(C0, 1e-6, 1.0 / 256, 1.0, 7)
    b = oracle.hyperdiffusion(C0, 1e-6, 1.0 / 256, 7)
    np.testing.assert_array_equal(a, b)


def _mode_factor(n, k, dt, dx, theta):
    """mu_k / lambda_k of the two circulant operators built from their fp64
    entries, evaluated in extended precision."""
    (e2, e1, e0), dg = oracle.hyperdiffusion_theta_operators(n, dt, dx, theta)
    a, b, c = (np.longdouble(v[0]) for v in dg[:3])
    th = 2 * np.pi * np.longdouble(k) / n
    lam = c + 2 * b * np.cos(th) + 2 * a * np.cos(2 * th)
    mu = np.longdouble(e0) + 2 * np.longdouble(e1) * np.cos(th) + 2 * np.longdouble(e2) * np.cos(2 * th)
    return mu / lam


@pytest.mark.parametrize("theta", [0.5, 0.25, 1.0])
@pytest.mark.parametrize("k", [1, 5, 16, 64])
def test_single_mode_factor(theta, k):
    """A cosine mode is an eigenvector of both operators: one step multiplies
    it by mu_k / lambda_k (for theta < 1/2 and high k the factor exceeds 1 in
    magnitude: the scheme is then unstable, which the oracle must reproduce)."""
    n, dt, dx = 256, 1e-6, 1.0 / 256
    x = np.arange(n) / n
    C0 = np.cos(2 * np.pi * k * x + 0.3)
    got = oracle.hyperdiffusion_theta(C0, dt, dx, theta, 1)[0]
    g = float(_mode_factor(n, k, dt, dx, theta))
    assert np.max(np.abs(got - g * C0)) <= 1e-11 * max(1.0, abs(g))


def test_mean_conserved():
    """sum(C) is the k = 0 component: multiplied by mu_0 / lambda_0 per step
    (1 up to the rounding of the entries).  The stencil entries (~2.6e4 at
    sigma = 4295) cancel to the O(1) mean, so each step may move it by
    ~eps * 2.6e4 relative: tolerance 1e-11 after 10 steps."""
    n, dt, dx, theta = 256, 1e-6, 1.0 / 256, 0.5
    rng = np.random.default_rng(11)
    C0 = rng.uniform(-1, 1, (4, n)) + 0.7
    got = oracle.hyperdiffusion_theta(C0, dt, dx, theta, 10)
    g0 = float(_mode_factor(n, 0, dt, dx, theta))
    np.testing.assert_allclose(got.sum(axis=1), C0.sum(axis=1) * g0 ** 10, rtol=1e-11)


@pytest.mark.parametrize("theta,order", [(0.5, 2.0), (1.0, 1.0)])
def test_temporal_order(theta, order):
    """Against the semi-discrete exact solution exp(-omega t) of a mode
    (omega = (2 - 2 cos(2 pi k / n))^2 / dx^4), halving dt divides the error
    at a fixed time by 2^order."""
    n, k, T = 32, 1, 2e-4
    dx = 1.0 / n
    x = np.arange(n) / n
    C0 = np.cos(2 * np.pi * k * x)
    omega = (2 - 2 * math.cos(2 * math.pi * k / n)) ** 2 / dx ** 4
    exact = math.exp(-omega * T) * C0
    errs = []
    for steps in (8, 16, 32):
        got = oracle.hyperdiffusion_theta(C0, T / steps, dx, theta, steps)[0]
        errs.append(np.max(np.abs(got - exact)))
    r1, r2 = errs[0] / errs[1], errs[1] / errs[2]
    for r in (r1, r2):
        assert abs(math.log2(r) - order) < 0.15, (errs, r1, r2)
