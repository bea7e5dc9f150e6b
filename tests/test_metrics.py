"""Pins of the comparator that gates every GPU parity assertion: hand-made
arrays whose errors are known exactly."""
import math

import numpy as np
import pytest

from oracle import max_rel_err, rel_err_p99, rel_err_p999, rel_err_pct


def test_exact_match_is_zero():
    r = np.array([[1.5, -2.0], [0.25, 8.0]])
    assert max_rel_err(r.copy(), r) == 0.0
    assert rel_err_p999(r.copy(), r) == 0.0


def test_known_offset():
    ref = np.array([1.0, -2.0, 4.0])
    out = ref + np.array([0.0, 0.04, 0.0])
    # the largest |difference| over the largest |reference|, not per element
    assert max_rel_err(out, ref) == pytest.approx(0.04 / 4.0, rel=1e-12)
    # a sign error on the largest element is a 200 % error
    assert max_rel_err(np.array([1.0, -2.0, -4.0]), ref) == pytest.approx(2.0, rel=1e-12)


def test_norm_wise_scale_hides_small_entries_but_p999_does_not():
    # 1 % of the entries are small (1e-2 of the maximum) and 100 % wrong
    ref = np.ones(10000)
    ref[:100] = 1e-2
    out = ref.copy()
    out[:100] = 0.0
    assert max_rel_err(out, ref) == pytest.approx(1e-2, rel=1e-12)   # passes a 2e-2 bar
    # element-wise: |0 - 1e-2| / (1e-2 + 1e-3) for 1 % > 0.1 % of the entries
    assert rel_err_p999(out, ref) == pytest.approx(1e-2 / 1.1e-2, rel=1e-12)


def test_p999_percentile_position():
    ref = np.ones(10000)
    few = ref.copy()
    few[:5] += 1.0            # 0.05 % of the entries: below the 99.9th percentile
    assert rel_err_p999(few, ref) == 0.0
    many = ref.copy()
    many[:20] += 1.0          # 0.2 %: the 99.9th percentile is one of them
    assert rel_err_p999(many, ref) == pytest.approx(1.0 / 1.001, rel=1e-12)


def test_p999_floor_relative_to_max():
    ref = np.zeros(1000)
    ref[0] = 1000.0
    out = ref.copy()
    out[1:] = 0.5             # absolute error 0.5 where ref = 0; floor is 1e-3 * 1000
    assert rel_err_p999(out, ref) == pytest.approx(0.5, rel=1e-12)
    assert max_rel_err(out, ref) == pytest.approx(0.5 / 1000.0, rel=1e-12)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_output_fails(bad):
    ref = np.array([1.0, 2.0, 3.0])
    out = ref.copy()
    out[1] = bad
    assert max_rel_err(out, ref) == math.inf
    assert rel_err_p999(out, ref) == math.inf
    assert not max_rel_err(out, ref) <= 1e9


def test_non_finite_reference_raises():
    with pytest.raises(ValueError):
        max_rel_err(np.zeros(2), np.array([1.0, np.nan]))
    with pytest.raises(ValueError):
        rel_err_p999(np.zeros(2), np.array([np.inf, 1.0]))


def test_zero_scale_falls_back_to_absolute():
    ref = np.zeros(4)
    assert max_rel_err(np.array([0.0, 1e-3, 0.0, -2e-3]), ref) == pytest.approx(2e-3)
    assert max_rel_err(np.zeros(4), ref) == 0.0
    assert rel_err_p999(np.zeros(4), ref) == 0.0


def test_shape_mismatch_raises():
    with pytest.raises(ValueError):
        max_rel_err(np.zeros((2, 3)), np.zeros((3, 2)))
    with pytest.raises(ValueError):
        rel_err_p999(np.zeros(5), np.zeros(6))


def test_empty_is_zero():
    assert max_rel_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0
    assert rel_err_p999(np.zeros(0), np.zeros(0)) == 0.0


def test_inputs_are_compared_in_float64():
    # a difference below float32 resolution of the values is still seen
    ref = np.array([1.0, 1.0], dtype=np.float64)
    out = np.array([1.0, 1.0 + 1e-12])
    assert max_rel_err(out, ref) == pytest.approx(1e-12, rel=1e-3)


def test_p99_position_and_general_percentile():
    ref = np.ones(10000)
    out = ref.copy()
    out[:50] += 1.0           # 0.5 %: below the 99th percentile, above the 99.9th
    assert rel_err_p99(out, ref) == 0.0
    assert rel_err_p999(out, ref) == pytest.approx(1.0 / 1.001, rel=1e-12)
    out[:200] += 1.0          # 2 %: both see it
    assert rel_err_p99(out, ref) > 0.9
    assert rel_err_pct(out, ref, 50.0) == 0.0
