"""Pins of the SSD and GLA forward oracles ("mlx-recurrence" post, Apple
Developer Forums thread 840535: ssd_scan with state [B, H, Dh, N]; gla_scan
with a scalar forget gate, an outer-product write and state [B, H, Dh, Dh])."""
import math

import numpy as np
import pytest

from oracle import diag_scan, gla_scan, selective_scan, ssd_scan


def _ssd_inputs(seed, Bn=2, L=12, H=4, P=3, G=2, N=5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bn, L, H, P))
    dt = np.log1p(np.exp(rng.normal(-1.0, 1.0, (Bn, L, H))))
    A = -np.exp(rng.uniform(0, math.log(16), H))
    Bm = rng.standard_normal((Bn, L, G, N))
    Cm = rng.standard_normal((Bn, L, G, N))
    Dk = rng.standard_normal(H)
    h0 = rng.standard_normal((Bn, H, P, N))
    return x, dt, A, Bm, Cm, Dk, h0


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_ssd_quadratic_unroll(disc):
    # y_t = sum_{s<=t} (C_t . B_s) prod_{r=s+1..t} e_r phi_s x_s
    #       + prod_{r<=t} e_r (h0 C_t) + D x_t      (head h reads group h//(H/G))
    x, dt, A, Bm, Cm, Dk, h0 = _ssd_inputs(20)
    y, hl, _ = ssd_scan(x, dt, A, Bm, Cm, Dk, h0, disc)
    Bn, L, H, P = x.shape
    G = Bm.shape[2]
    for b in range(Bn):
        for h in range(H):
            g = h // (H // G)
            lam = dt[b, :, h] * A[h]
            ph = np.expm1(lam) / A[h] if disc == "zoh" else dt[b, :, h]
            for t in range(L):
                ref = Dk[h] * x[b, t, h] + math.exp(lam[: t + 1].sum()) * (h0[b, h] @ Cm[b, t, g])
                for s in range(t + 1):
                    w = float(Cm[b, t, g] @ Bm[b, s, g]) * math.exp(lam[s + 1: t + 1].sum()) * ph[s]
                    ref = ref + w * x[b, s, h]
                np.testing.assert_allclose(y[b, t, h], ref, rtol=1e-11, atol=1e-11)


def test_ssd_is_selective_on_flattened_heads():
    # G = 1: SSD == selective scan with D = H*P channels, A[(h,p), n] = A[h],
    # dt[(h,p)] = dt[h], Dskip[(h,p)] = Dskip[h]
    x, dt, A, Bm, Cm, Dk, h0 = _ssd_inputs(21, G=1)
    Bn, L, H, P = x.shape
    N = Bm.shape[3]
    y, hl, _ = ssd_scan(x, dt, A, Bm, Cm, Dk, h0, "zoh")
    xs = x.reshape(Bn, L, H * P)
    dts = np.repeat(dt, P, axis=2)
    As = np.repeat(A, P)[:, None] * np.ones((1, N))
    ys, hls = selective_scan(xs, dts, As, Bm[:, :, 0], Cm[:, :, 0], np.repeat(Dk, P),
                             h0.reshape(Bn, H * P, N), "zoh")
    np.testing.assert_allclose(y.reshape(Bn, L, H * P), ys, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hl.reshape(Bn, H * P, N), hls, rtol=1e-12, atol=1e-12)


def test_ssd_groups_are_independent_head_sets():
    x, dt, A, Bm, Cm, Dk, h0 = _ssd_inputs(22, H=4, G=2)
    y, hl, _ = ssd_scan(x, dt, A, Bm, Cm, Dk, h0, "zoh")
    for g in range(2):
        hs = slice(2 * g, 2 * g + 2)
        yg, hlg, _ = ssd_scan(x[:, :, hs], dt[:, :, hs], A[hs], Bm[:, :, g:g + 1],
                              Cm[:, :, g:g + 1], Dk[hs], h0[:, hs], "zoh")
        np.testing.assert_allclose(y[:, :, hs], yg, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(hl[:, hs], hlg, rtol=1e-13, atol=1e-13)


def test_ssd_checkpoints_are_prefix_states():
    x, dt, A, Bm, Cm, Dk, h0 = _ssd_inputs(23, L=23)
    seg = 5
    y, hl, ck = ssd_scan(x, dt, A, Bm, Cm, Dk, h0, "zoh", seg=seg)
    assert ck.shape[0] == 5
    np.testing.assert_array_equal(ck[0], h0)
    for s in range(1, 5):
        _, hp, _ = ssd_scan(x[:, : s * seg], dt[:, : s * seg], A, Bm[:, : s * seg],
                            Cm[:, : s * seg], Dk, h0, "zoh")
        np.testing.assert_allclose(ck[s], hp, rtol=1e-13, atol=1e-13)
    # resuming from a checkpoint reproduces the rest of the sequence
    s0 = 3 * seg
    y2, hl2, _ = ssd_scan(x[:, s0:], dt[:, s0:], A, Bm[:, s0:], Cm[:, s0:], Dk, ck[3], "zoh")
    np.testing.assert_allclose(y2, y[:, s0:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hl2, hl, rtol=1e-12, atol=1e-12)


def _gla_inputs(seed, Bn=2, L=16, H=3, K=4, V=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Bn, L, H, K))
    k = rng.standard_normal((Bn, L, H, K))
    v = rng.standard_normal((Bn, L, H, V))
    g = 1.0 / (1.0 + np.exp(-rng.normal(1.0, 1.0, (Bn, L, H))))
    S0 = rng.standard_normal((Bn, H, K, V))
    return q, k, v, g, S0


def test_gla_unit_gate_is_causal_linear_attention():
    q, k, v, g, S0 = _gla_inputs(30)
    o, Sl = gla_scan(q, k, v, np.ones_like(g), S0)
    Bn, L, H, K = q.shape
    mask = np.tril(np.ones((L, L)))
    for b in range(Bn):
        for h in range(H):
            Q, Kt, Vv = q[b, :, h], k[b, :, h], v[b, :, h]
            ref = ((Q @ Kt.T) * mask) @ Vv + Q @ S0[b, h]
            np.testing.assert_allclose(o[b, :, h], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(Sl[b, h], S0[b, h] + Kt.T @ Vv, rtol=1e-12, atol=1e-12)


def test_gla_constant_gate_decay_mask():
    q, k, v, g, _ = _gla_inputs(31)
    gam = 0.8
    o, _ = gla_scan(q, k, v, np.full_like(g, gam))
    Bn, L, H, K = q.shape
    t = np.arange(L)
    Gm = np.where(t[:, None] >= t[None, :], gam ** (t[:, None] - t[None, :]), 0.0)
    for b in range(Bn):
        for h in range(H):
            ref = ((q[b, :, h] @ k[b, :, h].T) * Gm) @ v[b, :, h]
            np.testing.assert_allclose(o[b, :, h], ref, rtol=1e-12, atol=1e-12)


def test_gla_bruteforce_varying_gate():
    q, k, v, g, S0 = _gla_inputs(32, L=9)
    o, _ = gla_scan(q, k, v, g, S0)
    Bn, L, H, K = q.shape
    for b in range(Bn):
        for h in range(H):
            for t in range(L):
                ref = np.prod(g[b, : t + 1, h]) * (S0[b, h].T @ q[b, t, h])
                for s in range(t + 1):
                    w = np.prod(g[b, s + 1: t + 1, h]) * float(q[b, t, h] @ k[b, s, h])
                    ref = ref + w * v[b, s, h]
                np.testing.assert_allclose(o[b, t, h], ref, rtol=1e-12, atol=1e-12)


def test_gla_scalar_state_reduces_to_diag():
    q, k, v, g, S0 = _gla_inputs(33, K=1, V=1)
    o, Sl = gla_scan(q, k, v, g, S0)
    h, hl = diag_scan(g, k[..., 0] * v[..., 0], S0[:, :, 0, 0])
    np.testing.assert_allclose(o[..., 0], h * q[..., 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sl[:, :, 0, 0], hl, rtol=1e-12, atol=1e-12)
