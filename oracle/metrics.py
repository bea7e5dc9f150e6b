"""Error metrics used by the parity tests (test infrastructure only).

The pages ask only for a dtype-appropriate tolerance; the metric chosen is
the norm-wise maximum relative error of a whole output tensor,
    err = max|out - ref| / max|ref|,
with ``ref`` in float64.  Bars: <= 1e-4 for fp32 I/O, <= 2e-2 for bf16 I/O
with an fp32 state.  Element-wise figures,
    p99, p999 = 99th, 99.9th percentile of |out - ref| / (|ref| + 1e-3 max|ref|),
show errors on entries far below the tensor's maximum (small gradients,
early tokens) that the norm-wise figure cannot see.
"""
from __future__ import annotations

import numpy as np


def _pair(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise ValueError(f"shape mismatch {out.shape} vs {ref.shape}")
    if not np.all(np.isfinite(ref)):
        raise ValueError("reference holds non-finite values")
    return out, ref


def max_rel_err(out, ref) -> float:
    """max|out - ref| / max|ref|; the absolute difference when ref is all
    zero; inf when out holds a non-finite value; 0 for empty tensors."""
    out, ref = _pair(out, ref)
    if not np.all(np.isfinite(out)):
        return float("inf")
    if ref.size == 0:
        return 0.0
    scale = np.max(np.abs(ref))
    diff = np.max(np.abs(out - ref))
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)


def rel_err_pct(out, ref, q) -> float:
    """q-th percentile (numpy's linear interpolation) of
    |out - ref| / (|ref| + 1e-3 max|ref|); inf when out holds a non-finite
    value, 0 for empty tensors; with ref all zero the denominator is 1."""
    out, ref = _pair(out, ref)
    out, ref = out.ravel(), ref.ravel()
    if not np.all(np.isfinite(out)):
        return float("inf")
    if ref.size == 0:
        return 0.0
    s = 1e-3 * np.max(np.abs(ref))
    den = np.abs(ref) + (s if s > 0.0 else 1.0)
    return float(np.percentile(np.abs(out - ref) / den, q))


def rel_err_p999(out, ref) -> float:
    """rel_err_pct at the 99.9th percentile."""
    return rel_err_pct(out, ref, 99.9)


def rel_err_p99(out, ref) -> float:
    """rel_err_pct at the 99th percentile: entries whose reference is near
    zero by cancellation (sums of many terms of both signs) carry the
    operands' rounding at a large relative size, and 0.1 % of them can
    approach 50 % with bf16 operands; at the 99th percentile they stay well
    below it, while a mistake affecting 1 % of the entries shows."""
    return rel_err_pct(out, ref, 99.0)
