"""Pins of the SSD backward oracle ("mlx-recurrence" post, Apple Developer
Forums thread 840535: training with segment checkpointing and recompute).

The hand-derived adjoint in ``oracle.ssd_scan_bwd`` is checked against
torch.autograd (an independent library differentiation of a plain forward
loop), central finite differences and exact linearity identities."""
import math

import numpy as np
import pytest
import torch

from oracle import ssd_scan, ssd_scan_bwd


def _inputs(seed, Bn=2, L=9, H=4, P=3, G=2, N=4, A_zero_head=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bn, L, H, P))
    dt = np.log1p(np.exp(rng.normal(-1.0, 1.0, (Bn, L, H))))
    A = -np.exp(rng.uniform(0, math.log(16), H))
    if A_zero_head:
        A[1] = 0.0
        A[2] = -1e-7
    Bm = rng.standard_normal((Bn, L, G, N))
    Cm = rng.standard_normal((Bn, L, G, N))
    Dk = rng.standard_normal(H)
    h0 = rng.standard_normal((Bn, H, P, N))
    dy = rng.standard_normal((Bn, L, H, P))
    dhl = rng.standard_normal((Bn, H, P, N))
    return x, dt, A, Bm, Cm, Dk, h0, dy, dhl


def _torch_forward(x, dt, A, Bm, Cm, Dk, h0, disc):
    """Straight loop in torch fp64; only used to let autograd differentiate."""
    Bn, L, H, P = x.shape
    G = Bm.shape[2]
    Bh = Bm.repeat_interleave(H // G, dim=2)
    Ch = Cm.repeat_interleave(H // G, dim=2)
    h = h0
    ys = []
    for t in range(L):
        lam = dt[:, t] * A[None]
        e = torch.exp(lam)
        if disc == "zoh":
            # phi = dt * q(lam) with q(l) = expm1(l)/l (Taylor series near 0, so
            # that autograd also differentiates correctly at A == 0)
            small = lam.abs() < 1e-3
            safe = torch.where(small, torch.ones_like(lam), lam)
            q = torch.where(small, 1 + lam / 2 + lam ** 2 / 6 + lam ** 3 / 24 + lam ** 4 / 120,
                            torch.expm1(safe) / safe)
            phi = dt[:, t] * q
        else:
            phi = dt[:, t]
        h = e[..., None, None] * h + phi[..., None, None] * x[:, t, :, :, None] * Bh[:, t, :, None, :]
        ys.append((h * Ch[:, t, :, None, :]).sum(-1) + Dk[None, :, None] * x[:, t])
    return torch.stack(ys, 1), h


@pytest.mark.parametrize("disc", ["zoh", "euler"])
@pytest.mark.parametrize("zero_head", [False, True])
def test_bwd_matches_autograd(disc, zero_head):
    x, dt, A, Bm, Cm, Dk, h0, dy, dhl = _inputs(40, A_zero_head=zero_head)
    g = ssd_scan_bwd(x, dt, A, Bm, Cm, Dk, h0, dy, dhl, disc)
    T = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=Dk, h0=h0).items()}
    y, hl = _torch_forward(T["x"], T["dt"], T["A"], T["B"], T["C"], T["D"], T["h0"], disc)
    loss = (y * torch.tensor(dy)).sum() + (hl * torch.tensor(dhl)).sum()
    loss.backward()
    pairs = dict(dx="x", ddt="dt", dA="A", dB="B", dC="C", dD="D", dh0="h0")
    for mine, theirs in pairs.items():
        ref = T[theirs].grad.numpy()
        np.testing.assert_allclose(g[mine], ref, rtol=1e-9, atol=1e-9, err_msg=mine)


def test_bwd_finite_differences_dt_A():
    x, dt, A, Bm, Cm, Dk, h0, dy, dhl = _inputs(41, L=7)
    g = ssd_scan_bwd(x, dt, A, Bm, Cm, Dk, h0, dy, dhl, "zoh")

    def loss(dt_, A_):
        y, hl, _ = ssd_scan(x, dt_, A_, Bm, Cm, Dk, h0, "zoh")
        return float((y * dy).sum() + (hl * dhl).sum())

    eps = 1e-6
    for idx in [(0, 0, 0), (1, 3, 2), (0, 6, 3)]:
        dp, dm = dt.copy(), dt.copy()
        dp[idx] += eps
        dm[idx] -= eps
        fd = (loss(dp, A) - loss(dm, A)) / (2 * eps)
        assert abs(fd - g["ddt"][idx]) <= 1e-6 * (1 + abs(fd))
    for hh in range(A.shape[0]):
        Ap, Am = A.copy(), A.copy()
        Ap[hh] += eps
        Am[hh] -= eps
        fd = (loss(dt, Ap) - loss(dt, Am)) / (2 * eps)
        assert abs(fd - g["dA"][hh]) <= 1e-6 * (1 + abs(fd))


def test_bwd_linearity_identities():
    # With h0 = 0 the output is linear in x (and y - D x is linear in B and
    # in C), so <dy, y(x = v)> = <dx, v>, <dy, y(B = w) - D x> = <dB, w>,
    # <dy, y(C = w) - D x> = <dC, w>; and dD[h] = sum <dy, x>.
    x, dt, A, Bm, Cm, Dk, _, dy, _ = _inputs(42, L=11)
    rng = np.random.default_rng(43)
    g = ssd_scan_bwd(x, dt, A, Bm, Cm, Dk, None, dy, None, "zoh")
    v = rng.standard_normal(x.shape)
    yv, _, _ = ssd_scan(v, dt, A, Bm, Cm, Dk, None, "zoh")
    assert abs((dy * yv).sum() - (g["dx"] * v).sum()) < 1e-10
    w = rng.standard_normal(Bm.shape)
    yw, _, _ = ssd_scan(x, dt, A, w, Cm, Dk, None, "zoh")
    assert abs((dy * (yw - Dk[None, None, :, None] * x)).sum() - (g["dB"] * w).sum()) < 1e-10
    yc, _, _ = ssd_scan(x, dt, A, Bm, w, Dk, None, "zoh")
    assert abs((dy * (yc - Dk[None, None, :, None] * x)).sum() - (g["dC"] * w).sum()) < 1e-10
    np.testing.assert_allclose(g["dD"], np.einsum("blhp,blhp->h", dy, x), rtol=1e-13)
