"""Pins of the discretisations ("lrnnx: A library for Linear RNNs", Key
Contributions 2-3, which lists ZOH, bilinear and dirac among the schemes of
its fused selective-scan kernels; the pages give no formulas, the readings
are the textbook ones and are stated in oracle.discretize)."""
import numpy as np
import pytest
import scipy.signal

from oracle import discretize, discretize_grads, selective_scan


@pytest.mark.parametrize("method,disc", [("zoh", "zoh"), ("bilinear", "bilinear"),
                                         ("euler", "euler")])
def test_matches_scipy_cont2discrete(method, disc):
    # a diagonal continuous system, discretised by scipy's library routine
    rng = np.random.default_rng(0)
    N = 6
    A = -rng.uniform(0.1, 20.0, N)
    Bc = rng.standard_normal((N, 1))
    for dt in (1e-3, 0.05, 0.3, 2.0):
        ad, bd, *_ = scipy.signal.cont2discrete((np.diag(A), Bc, np.ones((1, N)), np.zeros((1, 1))),
                                                dt, method=method)
        e, phi = discretize(np.full(N, dt), A, disc)
        if disc != "euler":   # "euler" keeps the exact decay exp(dt A); only its input factor is Euler's
            np.testing.assert_allclose(np.diag(ad), e, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(bd[:, 0], phi * Bc[:, 0], rtol=1e-10, atol=1e-15)


def test_bilinear_steady_state_is_continuous_equilibrium():
    # constant dt, A < 0, B x: the fixed point of h = e h + phi B x is -B x / A
    # for both bilinear and ZOH (it does not depend on dt)
    A = np.array([[-0.7, -3.0]])
    for disc in ("bilinear", "zoh"):
        for dt in (0.01, 0.4):
            y, h = selective_scan(np.ones((1, 3000, 1)), np.full((1, 3000, 1), dt), A,
                                  np.full((1, 3000, 2), 2.0), np.zeros((1, 3000, 2)), h0=None,
                                  disc=disc)
            np.testing.assert_allclose(h[0, 0], -2.0 / A[0], rtol=1e-9)


def test_bilinear_is_pade_of_exp():
    # e(l) = (1 + l/2)/(1 - l/2) = exp(l) + l^3/12 + O(l^4)
    lam = np.array([1e-3, -2e-3, 5e-3])
    e, _ = discretize(lam, np.ones(3), "bilinear")
    np.testing.assert_allclose(e - np.exp(lam), lam ** 3 / 12, rtol=1e-2)


def test_bilinear_negative_decay_past_l_minus_2():
    e, phi = discretize(np.array([1.0]), np.array([-6.0]), "bilinear")
    assert e[0] == pytest.approx(-0.5) and phi[0] == pytest.approx(0.25)


def test_dirac_closed_forms():
    # phi = 1: constant inputs give h_t = B x (1 - e^{t+1}) / (1 - e); A = 0 gives cumsum(B x)
    L = 50
    dt, a = 0.3, -0.8
    y, h = selective_scan(np.ones((1, L, 1)) * 1.5, np.full((1, L, 1), dt), np.array([[a, 0.0]]),
                          np.tile([[[2.0, -1.0]]], (1, L, 1)), np.tile([[[1.0, 0.0]]], (1, L, 1)),
                          disc="dirac")
    e = np.exp(dt * a)
    t = np.arange(L)
    np.testing.assert_allclose(y[0, :, 0], 3.0 * (1 - e ** (t + 1)) / (1 - e), rtol=1e-12)
    np.testing.assert_allclose(h[0, 0, 1], -1.5 * L, rtol=1e-12)


@pytest.mark.parametrize("disc", ["bilinear", "dirac", "zoh", "euler"])
def test_grads_match_finite_differences(disc):
    rng = np.random.default_rng(1)
    dt = rng.uniform(0.01, 1.0, 7)
    A = -rng.uniform(0.1, 5.0, 7)
    e, phi = discretize(dt, A, disc)
    g = discretize_grads(dt, A, e, phi, disc)
    eps = 1e-7
    for k, (dd, dA) in enumerate(((eps, 0.0), (0.0, eps))):
        ep, pp = discretize(dt + dd, A + dA, disc)
        em, pm = discretize(dt - dd, A - dA, disc)
        np.testing.assert_allclose(g[k], (ep - em) / (2 * eps), rtol=1e-6, atol=1e-9)
        np.testing.assert_allclose(g[2 + k], (pp - pm) / (2 * eps), rtol=1e-6, atol=1e-9)
