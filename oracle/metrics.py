"""Error metrics used by the parity tests (test infrastructure only).

The pages ask only for a dtype-appropriate tolerance; the metric chosen is
the norm-wise maximum relative error of a whole output tensor,
    err = max|out - ref| / max|ref|,
with ``ref`` in float64.  Bars: <= 1e-4 for fp32 I/O, <= 2e-2 for bf16 I/O
with an fp32 state.
"""
from __future__ import annotations

import numpy as np


def max_rel_err(out, ref) -> float:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise ValueError(f"shape mismatch {out.shape} vs {ref.shape}")
    if not np.all(np.isfinite(out)):
        return float("inf")
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    diff = np.max(np.abs(out - ref)) if ref.size else 0.0
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)


def rel_err_p999(out, ref) -> float:
    """99.9th percentile of |out-ref| / (|ref| + 1e-3 max|ref|) (informative)."""
    out = np.asarray(out, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if ref.size == 0:
        return 0.0
    s = 1e-3 * np.max(np.abs(ref))
    return float(np.percentile(np.abs(out - ref) / (np.abs(ref) + s + 1e-300), 99.9))
