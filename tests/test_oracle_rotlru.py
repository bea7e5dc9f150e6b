"""Pins of the rotational-LRU oracle ("mlx-recurrence" post, rotlru_scan:
complex-diagonal recurrence with a magnitude gate and a per-step rotation of
two-dimensional channel pairs, state [B, D] as interleaved pairs)."""
import random

import numpy as np

from oracle import combine, diag_scan, rotlru_scan


def _rot(theta):
    c, s = np.cos(theta), np.sin(theta)
    return np.array([[c, -s], [s, c]])


def test_zero_angle_is_two_diagonal_scans():
    rng = np.random.default_rng(0)
    r = rng.uniform(0.5, 1.0, (2, 30, 3))
    u = rng.standard_normal((2, 30, 6))
    h0 = rng.standard_normal((2, 6))
    h, _ = rotlru_scan(r, np.zeros_like(r), u, h0)
    a = np.repeat(r, 2, axis=2)
    ref, _ = diag_scan(a, u, h0)
    np.testing.assert_allclose(h, ref, rtol=1e-13, atol=1e-13)


def test_matches_real_rotation_matrices():
    # each pair: h <- r R(theta) h + u with the 2x2 rotation matrix, written out
    rng = np.random.default_rng(1)
    L = 25
    r = rng.uniform(0.3, 1.0, (1, L, 2))
    th = rng.uniform(-np.pi, np.pi, (1, L, 2))
    u = rng.standard_normal((1, L, 4))
    h, _ = rotlru_scan(r, th, u)
    for p in range(2):
        v = np.zeros(2)
        for t in range(L):
            v = r[0, t, p] * _rot(th[0, t, p]) @ v + u[0, t, 2 * p:2 * p + 2]
            np.testing.assert_allclose(h[0, t, 2 * p:2 * p + 2], v, rtol=1e-12, atol=1e-12)


def test_constant_gate_and_angle_geometric_series():
    # z_t = w (1 - a^{t+1}) / (1 - a) with a = r e^{i theta}, z_{-1} = 0
    L, r, th = 80, 0.95, 0.3
    w = 0.7 - 1.1j
    u = np.zeros((1, L, 2))
    u[..., 0], u[..., 1] = w.real, w.imag
    h, _ = rotlru_scan(np.full((1, L, 1), r), np.full((1, L, 1), th), u)
    a = r * np.exp(1j * th)
    t = np.arange(L)
    z = w * (1 - a ** (t + 1)) / (1 - a)
    np.testing.assert_allclose(h[0, :, 0], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h[0, :, 1], z.imag, rtol=1e-12, atol=1e-12)


def test_unit_gate_preserves_norm_without_input():
    rng = np.random.default_rng(2)
    th = rng.uniform(-3, 3, (1, 50, 4))
    h0 = rng.standard_normal((1, 8))
    h, _ = rotlru_scan(np.ones_like(th), th, np.zeros((1, 50, 8)), h0)
    n0 = np.hypot(h0[0, 0::2], h0[0, 1::2])
    np.testing.assert_allclose(np.hypot(h[0, :, 0::2], h[0, :, 1::2]), np.tile(n0, (50, 1)), rtol=1e-12)


def test_complex_combine_associative():
    # the same combine, with complex (a, b), folded under random bracketings
    rng = np.random.default_rng(3)
    pairs = [(rng.uniform(0.5, 1) * np.exp(1j * rng.uniform(-3, 3)), complex(*rng.standard_normal(2)))
             for _ in range(17)]
    seq = pairs[0]
    for p in pairs[1:]:
        seq = combine(p, seq)
    for seed in range(5):
        items = list(pairs)
        rnd = random.Random(seed)
        while len(items) > 1:
            i = rnd.randrange(len(items) - 1)
            items[i:i + 2] = [combine(items[i + 1], items[i])]
        assert abs(items[0][0] - seq[0]) < 1e-12 and abs(items[0][1] - seq[1]) < 1e-12
