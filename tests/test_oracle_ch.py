"""Pins for the oracle's semi-implicit Cahn-Hilliard step (cuPentBatch page,
introduction: dC/dt = D d_xx (C^3 - C - gamma d_xx C), periodic, with the
phase-separation term taken at the old time level):

    (I + theta sigma D4) C^{k+1} = (I - (1-theta) sigma D4) C^k + r D2 (C^k^3 - C^k),
    r = D dt / dx^2,  sigma = gamma r / dx^2.

Independent checks: dense LAPACK solves on tiny grids; the linearised growth
factor of a small-amplitude Fourier mode about a constant state c0, which is
known in closed form and differs between a stable (|c0| > 1/sqrt 3) and a
spinodal (|c0| < 1/sqrt 3) background; mass conservation; constant states
being fixed points; convergence (first order in dt) to the semi-discrete
system integrated by an independent stiff ODE solver; the free energy of the
page's model decreasing along a trajectory."""
import math

import numpy as np
import pytest
from scipy.integrate import solve_ivp

import oracle
from dense import cyclic_dense, relerr


def _periodic_dense(n, taps):
    B = np.zeros((n, n))
    for i in range(n):
        for off, v in taps:
            B[i, (i + off) % n] += v
    return B


@pytest.mark.parametrize("n", [6, 7, 9, 16])
@pytest.mark.parametrize("theta", [0.5, 1.0, 0.3])
def test_matches_dense_lapack(n, theta):
    rng = np.random.default_rng(100 + n)
    dt, dx, gamma, mob = 2e-3, 1.0 / n, 0.05, 1.3
    (e2, e1, e0), r, dg = oracle.cahn_hilliard_operators(n, dt, dx, gamma, mob, theta)
    A = cyclic_dense(*dg)
    B = _periodic_dense(n, ((-2, e2), (-1, e1), (0, e0), (1, e1), (2, e2)))
    L2 = _periodic_dense(n, ((-1, 1.0), (0, -2.0), (1, 1.0)))
    C0 = rng.uniform(-1, 1, (3, n))
    got = oracle.cahn_hilliard(C0, dt, dx, gamma, mob, theta, 3)
    ref = C0.T.copy()
    for _ in range(3):
        ref = np.linalg.solve(A, B @ ref + r * (L2 @ (ref ** 3 - ref)))
    assert relerr(got, ref.T) < 1e-12


def _linear_factor(n, k, dt, dx, gamma, mob, theta, c0):
    """One-step amplification of mode k about C = c0 for the linearised scheme:
    (mu_k - r (3 c0^2 - 1) m_k) / lambda_k, m_k = 2 - 2 cos(2 pi k / n) (the
    symbol of -D2), evaluated from the rounded operator entries in extended
    precision."""
    (e2, e1, e0), r, dg = oracle.cahn_hilliard_operators(n, dt, dx, gamma, mob, theta)
    a, b, c = (np.longdouble(v[0]) for v in dg[:3])
    th = 2 * np.pi * np.longdouble(k) / n
    lam = c + 2 * b * np.cos(th) + 2 * a * np.cos(2 * th)
    mu = np.longdouble(e0) + 2 * np.longdouble(e1) * np.cos(th) + 2 * np.longdouble(e2) * np.cos(2 * th)
    m = 2 - 2 * np.cos(th)
    return float((mu - np.longdouble(r) * (3 * np.longdouble(c0) ** 2 - 1) * m) / lam)


@pytest.mark.parametrize("theta", [1.0, 0.5])
@pytest.mark.parametrize("c0", [0.0, 0.3, 0.8])
@pytest.mark.parametrize("k", [1, 5, 16])
def test_linearised_mode_factor(theta, c0, k):
    """C = c0 + eps cos(2 pi k x + 0.3): the k-th Fourier coefficient is
    multiplied by the linear factor up to O(eps^2) (the quadratic term feeds
    modes 0 and 2k only, the cubic one mode k at relative eps^2)."""
    n, dt, gamma, mob, eps = 64, 1e-5, 1e-3, 1.0, 1e-5
    dx = 1.0 / n
    x = np.arange(n) / n
    C0 = c0 + eps * np.cos(2 * np.pi * k * x + 0.3)
    C1 = oracle.cahn_hilliard(C0, dt, dx, gamma, mob, theta, 1)[0]
    ratio = np.fft.fft(C1)[k] / np.fft.fft(C0)[k]
    g = _linear_factor(n, k, dt, dx, gamma, mob, theta, c0)
    assert abs(ratio.imag) < 1e-8
    assert abs(ratio.real - g) < 1e-8, (ratio, g)


def test_spinodal_growth_and_stable_decay():
    """Inside the spinodal (c0 = 0) a long wave grows, outside (c0 = 0.8) it
    decays; the sign of the phase-separation term decides which."""
    n, dt, gamma, mob = 64, 1e-4, 1e-3, 1.0
    dx = 1.0 / n
    x = np.arange(n) / n
    for c0, grows in ((0.0, True), (0.8, False)):
        C0 = c0 + 1e-4 * np.cos(2 * np.pi * 2 * x)
        C1 = oracle.cahn_hilliard(C0, dt, dx, gamma, mob, 1.0, 20)[0]
        amp0, amp1 = np.abs(np.fft.fft(C0)[2]), np.abs(np.fft.fft(C1)[2])
        assert (amp1 > amp0) == grows, (c0, amp0, amp1)


def test_mass_conserved():
    """Both stencils and the implicit operator preserve the sum of C
    (D2 and D4 rows sum to zero)."""
    n, dt, gamma, mob = 128, 1e-5, 1e-3, 1.0
    rng = np.random.default_rng(5)
    C0 = rng.uniform(-0.5, 0.5, (4, n)) + 0.1
    got = oracle.cahn_hilliard(C0, dt, 1.0 / n, gamma, mob, 0.5, 25)
    np.testing.assert_allclose(got.sum(axis=1), C0.sum(axis=1), rtol=0, atol=1e-11)


@pytest.mark.parametrize("c0", [-1.0, 0.0, 0.37, 1.0])
def test_constant_state_is_fixed(c0):
    n = 32
    C0 = np.full((2, n), c0)
    got = oracle.cahn_hilliard(C0, 1e-4, 1.0 / n, 1e-2, 1.0, 1.0, 5)
    np.testing.assert_allclose(got, c0, rtol=0, atol=1e-14)


def _semidiscrete_rhs(n, dx, gamma, mob):
    L2 = _periodic_dense(n, ((-1, 1.0), (0, -2.0), (1, 1.0))) / dx ** 2
    L4 = L2 @ L2
    return lambda t, C: mob * (L2 @ (C ** 3 - C)) - gamma * mob * (L4 @ C)


@pytest.mark.parametrize("theta", [1.0, 0.5])
def test_first_order_convergence_to_semidiscrete(theta):
    """Against the method-of-lines system dC/dt = D L2 (C^3 - C) - gamma D L2^2 C
    integrated by scipy's Radau at tight tolerance: halving dt halves the error
    at a fixed time (the phase-separation term is explicit Euler)."""
    n, gamma, mob, T = 16, 1e-2, 1.0, 0.05
    dx = 1.0 / n
    x = np.arange(n) / n
    C0 = 0.1 * np.cos(2 * np.pi * x) + 0.05 * np.sin(4 * np.pi * x) + 0.02
    sol = solve_ivp(_semidiscrete_rhs(n, dx, gamma, mob), (0, T), C0, method="Radau",
                    rtol=1e-12, atol=1e-14)
    exact = sol.y[:, -1]
    assert np.max(np.abs(exact - C0)) > 0.05          # the state does evolve
    errs = []
    for steps in (40, 80, 160):
        got = oracle.cahn_hilliard(C0, T / steps, dx, gamma, mob, theta, steps)[0]
        errs.append(np.max(np.abs(got - exact)))
    for e_coarse, e_fine in zip(errs, errs[1:]):
        assert abs(math.log2(e_coarse / e_fine) - 1.0) < 0.15, errs


def test_free_energy_decreases():
    """The discrete free energy sum[(C^2 - 1)^2 / 4 + gamma/2 ((C_{i+1}-C_i)/dx)^2] dx
    of the page's model does not increase along a quench from a mixed state
    (small dt, theta = 1)."""
    n, gamma, mob, dt = 128, 1e-3, 1.0, 2e-6
    dx = 1.0 / n
    rng = np.random.default_rng(8)
    C = rng.uniform(-0.1, 0.1, (1, n))

    def energy(c):
        grad = (np.roll(c, -1) - c) / dx
        return float(np.sum(0.25 * (c ** 2 - 1) ** 2 + 0.5 * gamma * grad ** 2) * dx)

    E = [energy(C[0])]
    for _ in range(40):
        C = oracle.cahn_hilliard(C, dt, dx, gamma, mob, 1.0, 5)
        E.append(energy(C[0]))
    assert all(b <= a + 1e-13 for a, b in zip(E, E[1:])), E
    assert E[-1] < E[0] - 1e-3


def test_zero_nonlinear_limit_is_hyperdiffusion_theta():
    """With the phase-separation term switched off the linear part must be the
    theta-scheme hyperdiffusion step: for states of amplitude ~1e-7 the cubic
    part is negligible, and the -C part alone is a D2 term, so compare against
    hyperdiffusion_theta plus that correction solved densely."""
    n, dt, gamma, mob, theta = 32, 1e-5, 1e-2, 1.0, 0.5
    dx = 1.0 / n
    rng = np.random.default_rng(9)
    C0 = 1e-7 * rng.uniform(-1, 1, n)
    (e2, e1, e0), r, dg = oracle.cahn_hilliard_operators(n, dt, dx, gamma, mob, theta)
    A = cyclic_dense(*dg)
    L2 = _periodic_dense(n, ((-1, 1.0), (0, -2.0), (1, 1.0)))
    sigma = gamma * r / dx ** 2
    lin = oracle.hyperdiffusion_theta(C0, sigma * dx ** 4, dx, theta, 1)[0]
    corr = np.linalg.solve(A, -r * (L2 @ C0))
    got = oracle.cahn_hilliard(C0, dt, dx, gamma, mob, theta, 1)[0]
    assert np.max(np.abs(got - (lin + corr))) < 1e-12 * 1e-7 * 10
