"""Pins of the diagonal-recurrence oracle and the associative combine
(IBM Research blog "K-Search for MLX", section "A 20x faster prefill: the
Mamba SSM kernel": recurrence and combine equations)."""
import random

import numpy as np

from oracle import combine, diag_scan


def test_geometric_series_closed_form():
    # constant a, b and h_{-1} = 0:  h_t = b (1 - a^{t+1}) / (1 - a)
    L = 200
    a, b = 0.97, -1.3
    h, h_last = diag_scan(np.full((1, L, 1), a), np.full((1, L, 1), b))
    t = np.arange(L)
    ref = b * (1 - a ** (t + 1)) / (1 - a)
    np.testing.assert_allclose(h[0, :, 0], ref, rtol=1e-13, atol=1e-13)
    assert h_last[0, 0] == h[0, -1, 0]


def test_unit_decay_is_cumsum():
    rng = np.random.default_rng(0)
    b = rng.standard_normal((2, 50, 3))
    h, _ = diag_scan(np.ones_like(b), b)
    np.testing.assert_allclose(h, np.cumsum(b, axis=1), rtol=1e-13, atol=1e-12)


def test_zero_decay_is_identity():
    rng = np.random.default_rng(1)
    b = rng.standard_normal((2, 30, 4))
    h0 = rng.standard_normal((2, 4))
    h, _ = diag_scan(np.zeros_like(b), b, h0)
    np.testing.assert_array_equal(h, b)


def test_bruteforce_unroll():
    # h_t = prod_{r<=t} a_r h0 + sum_{s<=t} (prod_{r=s+1..t} a_r) b_s
    rng = np.random.default_rng(2)
    Bn, L, D = 2, 24, 3
    a = rng.uniform(-1.2, 1.2, (Bn, L, D))
    b = rng.standard_normal((Bn, L, D))
    h0 = rng.standard_normal((Bn, D))
    h, _ = diag_scan(a, b, h0)
    for bi in range(Bn):
        for d in range(D):
            for t in range(L):
                acc = h0[bi, d]
                for r in range(t + 1):
                    acc *= a[bi, r, d]
                for s in range(t + 1):
                    p = b[bi, s, d]
                    for r in range(s + 1, t + 1):
                        p *= a[bi, r, d]
                    acc += p
                assert abs(acc - h[bi, t, d]) <= 1e-12 * (1 + abs(acc))


def test_initial_state_linearity():
    rng = np.random.default_rng(3)
    a = rng.uniform(0.5, 1.0, (3, 40, 5))
    b = rng.standard_normal((3, 40, 5))
    h0 = rng.standard_normal((3, 5))
    h_with, _ = diag_scan(a, b, h0)
    h_without, _ = diag_scan(a, b)
    np.testing.assert_allclose(h_with, h_without + np.cumprod(a, axis=1) * h0[:, None, :],
                               rtol=1e-12, atol=1e-12)


def _fold(pairs, lo, hi, rnd):
    """Combine pairs[lo:hi] (earliest first) under a random bracketing."""
    if hi - lo == 1:
        return pairs[lo]
    mid = rnd.randint(lo + 1, hi - 1)
    left = _fold(pairs, lo, mid, rnd)      # earlier segment
    right = _fold(pairs, mid, hi, rnd)     # later segment
    return combine(right, left)


def test_combine_associative_any_bracketing():
    rng = np.random.default_rng(4)
    L = 64
    a = rng.uniform(0.8, 1.05, L)
    b = rng.standard_normal(L)
    h, _ = diag_scan(a[None, :, None], b[None, :, None])
    pairs = [(a[t], b[t]) for t in range(L)]
    rnd = random.Random(5)
    for _ in range(50):
        A_tot, B_tot = _fold(pairs, 0, L, rnd)
        # applied to h_{-1} = 0 the total pair gives h_{L-1}
        assert abs(B_tot - h[0, -1, 0]) <= 1e-12 * (1 + abs(B_tot))
        assert abs(A_tot - np.prod(a)) <= 1e-12 * abs(A_tot)
    # every prefix, random bracketing, with a non-zero initial state
    h0 = 0.7
    hh, _ = diag_scan(a[None, :, None], b[None, :, None], np.array([[h0]]))
    for t in range(1, L + 1):
        A_p, B_p = _fold(pairs, 0, t, rnd)
        assert abs(A_p * h0 + B_p - hh[0, t - 1, 0]) <= 1e-12 * (1 + abs(B_p))


def test_combine_not_commutative():
    p1, p2 = (0.5, 1.0), (2.0, 3.0)
    assert combine(p2, p1) == (1.0, 5.0)      # 2*1 + 3
    assert combine(p1, p2) == (1.0, 2.5)      # 0.5*3 + 1
