"""Pins of the GLA backward oracle ("mlx-recurrence" post, gla_scan: scalar
forget gate, outer-product write, state [B, H, Dh, Dh]; the training path of
the same post differentiates it)."""
import numpy as np
import torch

from oracle import gla_scan, gla_scan_bwd


def _case(seed, Bn=2, L=13, H=2, K=3, V=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Bn, L, H, K)) / np.sqrt(K)
    k = rng.standard_normal((Bn, L, H, K)) / np.sqrt(K)
    v = rng.standard_normal((Bn, L, H, V))
    g = rng.uniform(0.6, 1.0, (Bn, L, H))
    S0 = rng.standard_normal((Bn, H, K, V))
    do = rng.standard_normal((Bn, L, H, V))
    dSl = rng.standard_normal((Bn, H, K, V))
    return q, k, v, g, S0, do, dSl


def test_matches_autograd():
    q, k, v, g, S0, do, dSl = _case(0)
    T = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v, g, S0)]
    tq, tk, tv, tg, tS = T
    S = tS
    loss = 0.0
    for t in range(q.shape[1]):
        # plain loop over the recurrence, one (b, h) matrix product at a time
        S = tg[:, t, :, None, None] * S + tk[:, t, :, :, None] * tv[:, t, :, None, :]
        o = (S * tq[:, t, :, :, None]).sum(dim=2)
        loss = loss + (torch.tensor(do[:, t]) * o).sum()
    loss = loss + (torch.tensor(dSl) * S).sum()
    loss.backward()
    r = gla_scan_bwd(q, k, v, g, S0, do, dSl)
    for name, t in zip(("dq", "dk", "dv", "dg", "dS0"), T):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=1e-11, atol=1e-12, err_msg=name)


def test_finite_differences_gate():
    q, k, v, g, S0, do, dSl = _case(1, Bn=1, L=7, H=1)

    def loss(g_):
        o, Sl = gla_scan(q, k, v, g_, S0)
        return float((do * o).sum() + (dSl * Sl).sum())

    r = gla_scan_bwd(q, k, v, g, S0, do, dSl)
    eps = 1e-6
    for t in (0, 3, 6):
        gp, gm = g.copy(), g.copy()
        gp[0, t, 0] += eps
        gm[0, t, 0] -= eps
        assert abs((loss(gp) - loss(gm)) / (2 * eps) - r["dg"][0, t, 0]) < 1e-7


def test_linearity_identities():
    # o is linear in q; with S0 = 0 it is linear in v and in k separately
    q, k, v, g, _, do, _ = _case(2, Bn=2, L=40, H=2, K=4, V=5)
    w = np.random.default_rng(3)
    r = gla_scan_bwd(q, k, v, g, None, do)
    wq = w.standard_normal(q.shape)
    o, _ = gla_scan(wq, k, v, g)
    assert abs((do * o).sum() - (r["dq"] * wq).sum()) < 1e-9
    wv = w.standard_normal(v.shape)
    o, _ = gla_scan(q, k, wv, g)
    assert abs((do * o).sum() - (r["dv"] * wv).sum()) < 1e-9
    wk = w.standard_normal(k.shape)
    o, _ = gla_scan(q, wk, v, g)
    assert abs((do * o).sum() - (r["dk"] * wk).sum()) < 1e-9


def test_unit_gate_is_causal_linear_attention_grad():
    # g = 1, S0 = 0: O = tril(Q K^T) V per (b, h); dV = tril(Q K^T)^T dO
    q, k, v, _, _, do, _ = _case(4, Bn=1, L=20, H=1, K=3, V=2)
    g = np.ones(q.shape[:3])
    r = gla_scan_bwd(q, k, v, g, None, do)
    Q, Kk, dO = q[0, :, 0], k[0, :, 0], do[0, :, 0]
    Amat = np.tril(Q @ Kk.T)
    np.testing.assert_allclose(r["dv"][0, :, 0], Amat.T @ dO, rtol=1e-12, atol=1e-12)
    dA = np.tril(dO @ v[0, :, 0].T)
    np.testing.assert_allclose(r["dq"][0, :, 0], dA @ Kk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dk"][0, :, 0], dA.T @ Q, rtol=1e-12, atol=1e-12)
