"""Pins of the Mamba-1 selective-scan oracle ("lrnnx: A library for Linear
RNNs", Key Contributions 2-3: ZOH discretisation, fused scan + output
projection)."""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import diag_scan, discretize, selective_scan


def _rand(seed, Bn=2, L=20, D=3, N=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bn, L, D))
    dt = np.log1p(np.exp(rng.normal(-1.0, 1.0, (Bn, L, D))))
    A = -rng.uniform(0.2, 3.0, (D, N))
    Bm = rng.standard_normal((Bn, L, N))
    Cm = rng.standard_normal((Bn, L, N))
    Dk = rng.standard_normal(D)
    h0 = rng.standard_normal((Bn, D, N))
    return x, dt, A, Bm, Cm, Dk, h0


def test_zoh_matches_matrix_exponential():
    # Exact ZOH of dh/dtau = A h + u over a step dt with constant u is the
    # top-right block of expm([[A dt, u dt], [0, 0]]) (Van Loan); scipy's expm
    # is the independent library routine.
    rng = np.random.default_rng(10)
    for _ in range(20):
        A = -rng.uniform(0.01, 5.0)
        dt = rng.uniform(0.001, 2.0)
        M = np.array([[A * dt, dt], [0.0, 0.0]])
        E = scipy.linalg.expm(M)
        e, phi = discretize(np.array(dt), np.array(A), "zoh")
        # scipy's expm (scaling and squaring) is accurate to ~1e-12 relative
        assert abs(e - E[0, 0]) <= 1e-12 * abs(E[0, 0])
        assert abs(phi - E[0, 1]) <= 1e-12 * abs(E[0, 1])


def test_zoh_tiny_and_zero_A():
    e, phi = discretize(np.array([0.3, 0.3, 0.3]), np.array([0.0, 1e-12, -1e-12]), "zoh")
    np.testing.assert_allclose(phi, [0.3, 0.3, 0.3], rtol=1e-11)
    np.testing.assert_allclose(e, [1.0, 1.0, 1.0], rtol=1e-11)


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_steady_state_closed_form(disc):
    # constant dt, A<0, B, x, h_{-1}=0: h_t = phi B x (1 - e^{t+1}) / (1 - e).
    # For ZOH this is (-B x / A)(1 - e^{t+1}): the continuous-time equilibrium
    # -Bx/A, independent of dt; Euler's limit dt B x / (1 - e) depends on dt.
    L, dtv, Av, Bv, xv = 300, 0.05, -2.0, 0.7, 1.3
    x = np.full((1, L, 1), xv)
    dt = np.full((1, L, 1), dtv)
    A = np.full((1, 1), Av)
    Bm = np.full((1, L, 1), Bv)
    Cm = np.ones((1, L, 1))
    y, _ = selective_scan(x, dt, A, Bm, Cm, None, None, disc)
    e = math.exp(dtv * Av)
    t = np.arange(L)
    if disc == "zoh":
        ref = (-Bv * xv / Av) * (1 - e ** (t + 1))
    else:
        ref = dtv * Bv * xv * (1 - e ** (t + 1)) / (1 - e)
    np.testing.assert_allclose(y[0, :, 0], ref, rtol=1e-12, atol=1e-13)


def test_A_zero_is_cumsum():
    x, dt, A, Bm, Cm, Dk, _ = _rand(11)
    A = np.zeros_like(A)
    y, _ = selective_scan(x, dt, A, Bm, Cm, Dk, None, "zoh")
    # h_t[d,n] = sum_{s<=t} dt_s[d] B_s[n] x_s[d]
    h = np.cumsum(dt[:, :, :, None] * Bm[:, :, None, :] * x[:, :, :, None], axis=1)
    ref = np.einsum("bldn,bln->bld", h, Cm) + Dk * x
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_bruteforce_unroll(disc):
    x, dt, A, Bm, Cm, Dk, h0 = _rand(12, Bn=2, L=10, D=2, N=3)
    y, hl = selective_scan(x, dt, A, Bm, Cm, Dk, h0, disc)
    Bn, L, D = x.shape
    N = A.shape[1]
    for b in range(Bn):
        for d in range(D):
            for t in range(L):
                acc = Dk[d] * x[b, t, d]
                for n in range(N):
                    lam = [dt[b, r, d] * A[d, n] for r in range(L)]
                    if disc == "zoh":
                        ph = [math.expm1(lam[r]) / A[d, n] for r in range(L)]
                    else:
                        ph = [dt[b, r, d] for r in range(L)]
                    hn = h0[b, d, n] * math.exp(sum(lam[: t + 1]))
                    for s in range(t + 1):
                        hn += math.exp(sum(lam[s + 1: t + 1])) * ph[s] * Bm[b, s, n] * x[b, s, d]
                    acc += Cm[b, t, n] * hn
                assert abs(acc - y[b, t, d]) <= 1e-11 * (1 + abs(acc))


def test_single_channel_reduces_to_diag():
    x, dt, A, Bm, Cm, Dk, h0 = _rand(13, Bn=2, L=40, D=1, N=1)
    y, hl = selective_scan(x, dt, A, Bm, Cm, None, h0, "zoh")
    e, phi = discretize(dt, A[0, 0], "zoh")
    h, hl2 = diag_scan(e, phi * Bm * x, h0[:, :, 0])
    np.testing.assert_allclose(y, h * Cm, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hl[:, :, 0], hl2, rtol=1e-12, atol=1e-12)
