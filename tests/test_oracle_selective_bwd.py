"""Pins of the Mamba-1 selective-scan backward oracle ("lrnnx: A library for
Linear RNNs", Key Contributions 2-3: time-varying selective scan with ZOH and
a fused readout; its gradients are what a training path needs)."""
import numpy as np
import pytest
import torch

from oracle import selective_scan, selective_scan_bwd, ssd_scan_bwd


def _case(seed, Bn=2, L=11, D=3, N=4, zero_A=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bn, L, D))
    dt = np.log1p(np.exp(rng.normal(-1.0, 0.5, (Bn, L, D))))
    A = -rng.uniform(0.2, 3.0, (D, N))
    if zero_A:
        A[0, :2] = 0.0
        A[1, 1] = -1e-5
    Bm = rng.standard_normal((Bn, L, N))
    Cm = rng.standard_normal((Bn, L, N))
    Dk = rng.standard_normal(D)
    h0 = rng.standard_normal((Bn, D, N))
    dy = rng.standard_normal((Bn, L, D))
    dhl = rng.standard_normal((Bn, D, N))
    return x, dt, A, Bm, Cm, Dk, h0, dy, dhl


def _torch_grads(x, dt, A, Bm, Cm, Dk, h0, dy, dhl, disc):
    """autograd over an independent plain loop; the ZOH input factor uses the
    series dt (1 + l/2 + l^2/6 + l^3/24 + l^4/120) near l = dt A = 0."""
    T = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, dt, A, Bm, Cm, Dk, h0)]
    tx, tdt, tA, tB, tC, tD, th = T
    loss = 0.0
    for t in range(x.shape[1]):
        lam = tdt[:, t, :, None] * tA[None]
        e = torch.exp(lam)
        if disc == "zoh":
            ser = 1 + lam / 2 + lam ** 2 / 6 + lam ** 3 / 24 + lam ** 4 / 120
            q = torch.where(lam.abs() < 1e-3, ser, torch.expm1(lam) / torch.where(lam == 0, 1.0, lam))
            phi = tdt[:, t, :, None] * q
        elif disc == "bilinear":
            e = (1 + lam / 2) / (1 - lam / 2)
            phi = tdt[:, t, :, None] / (1 - lam / 2)
        elif disc == "dirac":
            phi = torch.ones_like(lam)
        else:
            phi = tdt[:, t, :, None].expand_as(lam)
        th = e * th + phi * tB[:, t, None, :] * tx[:, t, :, None]
        y = (th * tC[:, t, None, :]).sum(-1) + tD * tx[:, t]
        loss = loss + (torch.tensor(dy[:, t]) * y).sum()
    loss = loss + (torch.tensor(dhl) * th).sum()
    loss.backward()
    return [t.grad.numpy() for t in T]


@pytest.mark.parametrize("disc", ["zoh", "euler", "bilinear", "dirac"])
@pytest.mark.parametrize("zero_A", [False, True])
def test_matches_autograd(disc, zero_A):
    c = _case(0, zero_A=zero_A)
    r = selective_scan_bwd(*c[:7], c[7], c[8], disc)
    g = _torch_grads(*c, disc)
    for name, ref in zip(("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"), g):
        np.testing.assert_allclose(r[name], ref, rtol=1e-9, atol=1e-10, err_msg=name)


def test_finite_differences_dt_A():
    x, dt, A, Bm, Cm, Dk, h0, dy, dhl = _case(1, Bn=1, L=6, D=2, N=3)

    def loss(dt_, A_):
        y, hl = selective_scan(x, dt_, A_, Bm, Cm, Dk, h0)
        return float((dy * y).sum() + (dhl * hl).sum())

    r = selective_scan_bwd(x, dt, A, Bm, Cm, Dk, h0, dy, dhl)
    eps = 1e-6
    for idx in [(0, 0, 0), (0, 3, 1), (0, 5, 1)]:
        p, m = dt.copy(), dt.copy()
        p[idx] += eps
        m[idx] -= eps
        assert abs((loss(p, A) - loss(m, A)) / (2 * eps) - r["ddt"][idx]) < 1e-6
    for idx in [(0, 0), (1, 2)]:
        p, m = A.copy(), A.copy()
        p[idx] += eps
        m[idx] -= eps
        assert abs((loss(dt, p) - loss(dt, m)) / (2 * eps) - r["dA"][idx]) < 1e-6


def test_linearity_identities():
    # y is linear in x (h0 = 0); y - D x is linear in B and in C
    x, dt, A, Bm, Cm, Dk, _, dy, _ = _case(2, Bn=2, L=50, D=4, N=5)
    r = selective_scan_bwd(x, dt, A, Bm, Cm, Dk, None, dy)
    w = np.random.default_rng(3)
    v = w.standard_normal(x.shape)
    y, _ = selective_scan(v, dt, A, Bm, Cm, Dk)
    assert abs((dy * y).sum() - (r["dx"] * v).sum()) < 1e-9 * max(1, abs((dy * y).sum()))
    v = w.standard_normal(Bm.shape)
    y, _ = selective_scan(x, dt, A, v, Cm, None)
    assert abs((dy * y).sum() - (r["dB"] * v).sum()) < 1e-9 * max(1, abs((dy * y).sum()))
    v = w.standard_normal(Cm.shape)
    y, _ = selective_scan(x, dt, A, Bm, v, None)
    assert abs((dy * y).sum() - (r["dC"] * v).sum()) < 1e-9 * max(1, abs((dy * y).sum()))
    np.testing.assert_allclose(r["dD"], np.einsum("bld,bld->d", dy, x), rtol=1e-12)


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_cross_check_with_ssd_backward(disc):
    """An SSD head with P = 1 and G = 1 is a selective-scan channel whose A row
    is constant: both independently written adjoints must agree."""
    x, dt, _, Bm, Cm, Dk, h0, dy, dhl = _case(4, Bn=2, L=20, D=3, N=4)
    Ah = -np.array([0.5, 1.5, 2.5])
    A = np.repeat(Ah[:, None], 4, axis=1)
    r = selective_scan_bwd(x, dt, A, Bm, Cm, Dk, h0, dy, dhl, disc)
    s = ssd_scan_bwd(x[..., None], dt, Ah, Bm[:, :, None], Cm[:, :, None], Dk, h0[:, :, None],
                     dy[..., None], dhl[:, :, None], disc)
    np.testing.assert_allclose(r["dx"], s["dx"][..., 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["ddt"], s["ddt"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dA"].sum(axis=1), s["dA"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dB"], s["dB"][:, :, 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dC"], s["dC"][:, :, 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["dh0"], s["dh0"][:, :, 0], rtol=1e-10, atol=1e-12)
