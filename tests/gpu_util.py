"""Helpers for the GPU parity tests: upload seeded inputs, compare with the
oracle under the norm-wise max relative error bar, and report the
element-wise 99th- and 99.9th-percentile errors beside it under bars of
their own (they catch small entries that are wrong by a large factor, which
the norm-wise figure scales away)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import max_rel_err, rel_err_pct

TOL = {"f32": 1e-4, "bf16": 2e-2}
# bars of the element-wise figures (99th and 99.9th percentile of
# |out - ref| / (|ref| + 1e-3 max|ref|)), by the norm-wise bar they go with.
# Measured worst cases over the GPU suite: fp32 p999 4.2e-4; bf16 p999 0.50
# (dC and dk: sums of 2048 bf16-operand products, whose near-zero entries
# come from cancellation), hence the 99th percentile as the bf16 gate.
P99_TOL = {1e-4: 2.5e-3, 2e-2: 2.5e-1}
P999_TOL = {1e-4: 5e-3, 2e-2: 1.0}


def dev(t, io=None):
    """numpy float32 (bf16-representable when io == 'bf16') -> cuda tensor."""
    arr = t.values if hasattr(t, "values") else t
    io = io or (t.io if hasattr(t, "io") else "f32")
    x = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    return x.to(torch.bfloat16) if io == "bf16" else x


def host(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def check(name, out, ref, tol, log=None):
    o = host(out) if torch.is_tensor(out) else out
    err = max_rel_err(o, ref)
    p99, p999 = rel_err_pct(o, ref, 99.0), rel_err_pct(o, ref, 99.9)
    t99, t999 = P99_TOL.get(tol, 25.0 * tol), P999_TOL.get(tol, 50.0 * tol)
    msg = (f"{name}: max_rel_err={err:.3e} (tol {tol:.1e}) p99={p99:.3e} (tol {t99:.1e}) "
           f"p999={p999:.3e} (tol {t999:.1e})")
    print(msg, flush=True)
    if log is not None:
        log.append((name, err, p99, p999))
    assert err <= tol, msg
    assert p99 <= t99, msg
    assert p999 <= t999, msg
    return err
