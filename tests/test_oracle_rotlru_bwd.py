"""Pins of the rotational-LRU backward oracle (reverse-time adjoint of the
complex-diagonal recurrence over channel pairs; "mlx-recurrence" post, Apple
Developer Forums thread 840535, rotlru_scan, whose kernel has a forward and a
backward)."""
import numpy as np
import torch

from oracle import diag_scan, diag_scan_bwd, rotlru_scan, rotlru_scan_bwd


def _case(seed, Bn=2, L=23, P=3):
    rng = np.random.default_rng(seed)
    r = rng.uniform(0.4, 1.05, (Bn, L, P))
    th = rng.uniform(-np.pi, np.pi, (Bn, L, P))
    u = rng.standard_normal((Bn, L, 2 * P))
    h0 = rng.standard_normal((Bn, 2 * P))
    dh = rng.standard_normal((Bn, L, 2 * P))
    dhl = rng.standard_normal((Bn, 2 * P))
    return r, th, u, h0, dh, dhl


def _torch_grads(r, th, u, h0, dh, dhl):
    """torch.autograd (fp64, CPU) through the real 2x2 form of each step,
    h <- r [[cos, -sin], [sin, cos]] h + u, written independently."""
    tr, tth, tu, th0 = (torch.tensor(v, dtype=torch.float64, requires_grad=True)
                        for v in (r, th, u, h0))
    x, y = th0[:, 0::2], th0[:, 1::2]
    loss = 0.0
    for t in range(r.shape[1]):
        c, s = torch.cos(tth[:, t]), torch.sin(tth[:, t])
        x, y = (tr[:, t] * (c * x - s * y) + tu[:, t, 0::2],
                tr[:, t] * (s * x + c * y) + tu[:, t, 1::2])
        loss = loss + (torch.tensor(dh[:, t, 0::2]) * x).sum() + (torch.tensor(dh[:, t, 1::2]) * y).sum()
    loss = loss + (torch.tensor(dhl[:, 0::2]) * x).sum() + (torch.tensor(dhl[:, 1::2]) * y).sum()
    loss.backward()
    return tr.grad.numpy(), tth.grad.numpy(), tu.grad.numpy(), th0.grad.numpy()


def test_matches_autograd_of_rotation_matrices():
    r, th, u, h0, dh, dhl = _case(0)
    h, _ = rotlru_scan(r, th, u, h0)
    got = rotlru_scan_bwd(r, th, h, dh, h0, dhl)
    ref = _torch_grads(r, th, u, h0, dh, dhl)
    for name, g, e in zip(("dr", "dtheta", "du", "dh0"), got, ref):
        np.testing.assert_allclose(g, e, rtol=1e-11, atol=1e-11, err_msg=name)


def test_finite_differences():
    r, th, u, h0, dh, dhl = _case(1, Bn=1, L=7, P=2)

    def loss(r_, th_, u_, h0_):
        h, hl = rotlru_scan(r_, th_, u_, h0_)
        return float((dh * h).sum() + (dhl * hl).sum())

    h, _ = rotlru_scan(r, th, u, h0)
    dr, dth, du, dh0 = rotlru_scan_bwd(r, th, h, dh, h0, dhl)
    eps = 1e-6
    args = [r, th, u, h0]
    for k, grad, idxs in ((0, dr, [(0, 0, 0), (0, 3, 1), (0, 6, 0)]),
                          (1, dth, [(0, 0, 1), (0, 4, 0), (0, 6, 1)]),
                          (2, du, [(0, 0, 3), (0, 5, 0), (0, 6, 2)]),
                          (3, dh0, [(0, 0), (0, 3)])):
        for idx in idxs:
            p = [a.copy() for a in args]
            m = [a.copy() for a in args]
            p[k][idx] += eps
            m[k][idx] -= eps
            fd = (loss(*p) - loss(*m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(fd)), (k, idx, fd, grad[idx])


def test_zero_angle_reduces_to_diagonal_backward():
    # theta = 0: both halves of a pair run the real diagonal recurrence with
    # the gate r, so du is db and dr is the sum of the pair's da
    r, _, u, h0, dh, dhl = _case(2)
    th = np.zeros_like(r)
    h, _ = rotlru_scan(r, th, u, h0)
    dr, dth, du, dh0 = rotlru_scan_bwd(r, th, h, dh, h0, dhl)
    a = np.repeat(r, 2, axis=2)
    hd, _ = diag_scan(a, u, h0)
    da, db, rdh0 = diag_scan_bwd(a, hd, dh, h0, dhl)
    np.testing.assert_allclose(du, db, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dh0, rdh0, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dr, da[..., 0::2] + da[..., 1::2], rtol=1e-12, atol=1e-12)


def test_rotation_invariance_of_theta_gradient():
    # rotating every state and input pair by a fixed angle phi leaves the
    # dynamics equivariant; for a loss read out along the rotated frame
    # the theta gradient is unchanged (a check on signs in dtheta)
    r, th, u, h0, dh, dhl = _case(3, Bn=1, L=15, P=2)

    def rot(v, phi):
        z = (v[..., 0::2] + 1j * v[..., 1::2]) * np.exp(1j * phi)
        out = np.empty_like(v)
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
        return out

    h, _ = rotlru_scan(r, th, u, h0)
    g0 = rotlru_scan_bwd(r, th, h, dh, h0, dhl)
    phi = 0.83
    hr, _ = rotlru_scan(r, th, rot(u, phi), rot(h0, phi))
    np.testing.assert_allclose(hr, rot(h, phi), rtol=1e-12, atol=1e-12)
    g1 = rotlru_scan_bwd(r, th, hr, rot(dh, phi), rot(h0, phi), rot(dhl, phi))
    np.testing.assert_allclose(g1[0], g0[0], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g1[1], g0[1], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g1[2], rot(g0[2], phi), rtol=1e-11, atol=1e-11)


def test_empty_sequence_passes_dh_last():
    z = np.zeros((2, 0, 3))
    dhl = np.arange(12.0).reshape(2, 6)
    dr, dth, du, dh0 = rotlru_scan_bwd(z, z, np.zeros((2, 0, 6)), np.zeros((2, 0, 6)), None, dhl)
    assert dr.shape == (2, 0, 3) and du.shape == (2, 0, 6)
    np.testing.assert_array_equal(dh0, dhl)
