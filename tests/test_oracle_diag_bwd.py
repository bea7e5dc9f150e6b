"""Pins of the diagonal-recurrence backward oracle (reverse-time adjoint of
h_t = a_t h_{t-1} + b_t; IBM Research blog "K-Search for MLX", section "A 20x
faster prefill: the Mamba SSM kernel", recurrence equation; the gradients of
a trained recurrence are what the "mlx-recurrence" post's training path
computes)."""
import numpy as np
import torch

from oracle import diag_scan, diag_scan_bwd


def _torch_loss_grads(a, b, h0, dh, dh_last):
    """torch.autograd over a plain loop (fp64, CPU), written independently."""
    ta = torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tb = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    th0 = torch.tensor(h0, dtype=torch.float64, requires_grad=True)
    state = th0
    loss = 0.0
    for t in range(a.shape[1]):
        state = ta[:, t] * state + tb[:, t]
        loss = loss + (torch.tensor(dh[:, t]) * state).sum()
    loss = loss + (torch.tensor(dh_last) * state).sum()
    loss.backward()
    return ta.grad.numpy(), tb.grad.numpy(), th0.grad.numpy()


def _case(seed, Bn=2, L=37, D=3):
    rng = np.random.default_rng(seed)
    a = rng.uniform(0.5, 1.1, (Bn, L, D))
    b = rng.standard_normal((Bn, L, D))
    h0 = rng.standard_normal((Bn, D))
    dh = rng.standard_normal((Bn, L, D))
    dh_last = rng.standard_normal((Bn, D))
    return a, b, h0, dh, dh_last


def test_matches_autograd():
    a, b, h0, dh, dhl = _case(0)
    h, _ = diag_scan(a, b, h0)
    da, db, dh0 = diag_scan_bwd(a, h, dh, h0, dhl)
    ra, rb, rh0 = _torch_loss_grads(a, b, h0, dh, dhl)
    np.testing.assert_allclose(da, ra, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db, rb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dh0, rh0, rtol=1e-12, atol=1e-12)


def test_finite_differences():
    a, b, h0, dh, dhl = _case(1, Bn=1, L=9, D=2)

    def loss(a_, b_, h0_):
        h, hl = diag_scan(a_, b_, h0_)
        return float((dh * h).sum() + (dhl * hl).sum())

    h, _ = diag_scan(a, b, h0)
    da, db, dh0 = diag_scan_bwd(a, h, dh, h0, dhl)
    eps = 1e-6
    for idx in [(0, 0, 0), (0, 4, 1), (0, 8, 0)]:
        ap, am = a.copy(), a.copy()
        ap[idx] += eps
        am[idx] -= eps
        assert abs((loss(ap, b, h0) - loss(am, b, h0)) / (2 * eps) - da[idx]) < 1e-7
        bp, bm = b.copy(), b.copy()
        bp[idx] += eps
        bm[idx] -= eps
        assert abs((loss(a, bp, h0) - loss(a, bm, h0)) / (2 * eps) - db[idx]) < 1e-7
    hp, hm = h0.copy(), h0.copy()
    hp[0, 1] += eps
    hm[0, 1] -= eps
    assert abs((loss(a, b, hp) - loss(a, b, hm)) / (2 * eps) - dh0[0, 1]) < 1e-7


def test_unit_decay_is_reverse_cumsum():
    # a = 1: g_t = sum_{s >= t} dh_s (+ dh_last)
    rng = np.random.default_rng(2)
    dh = rng.standard_normal((2, 40, 3))
    dhl = rng.standard_normal((2, 3))
    a = np.ones_like(dh)
    h, _ = diag_scan(a, rng.standard_normal(dh.shape))
    _, db, dh0 = diag_scan_bwd(a, h, dh, None, dhl)
    ref = np.cumsum(dh[:, ::-1], axis=1)[:, ::-1] + dhl[:, None]
    np.testing.assert_allclose(db, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dh0, ref[:, 0], rtol=1e-12, atol=1e-12)


def test_linearity_in_b():
    # h is linear in (b, h0): <dh, h(b=v, h0=0)> + <dh_last, h_last> = <db, v>
    a, _, _, dh, dhl = _case(3, Bn=2, L=64, D=5)
    v = np.random.default_rng(4).standard_normal(a.shape)
    h, hl = diag_scan(a, v)
    _, db, _ = diag_scan_bwd(a, h, dh, None, dhl)
    lhs = (dh * h).sum() + (dhl * hl).sum()
    assert abs(lhs - (db * v).sum()) <= 1e-10 * max(1.0, abs(lhs))


def test_empty_sequence_passes_dh_last():
    dhl = np.arange(6.0).reshape(2, 3)
    z = np.zeros((2, 0, 3))
    da, db, dh0 = diag_scan_bwd(z, z, z, None, dhl)
    assert da.shape == (2, 0, 3) and db.shape == (2, 0, 3)
    np.testing.assert_array_equal(dh0, dhl)
