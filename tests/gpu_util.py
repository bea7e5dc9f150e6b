"""Helpers for the GPU parity tests: upload seeded inputs, compare with the
oracle under the norm-wise max relative error bar, and report the
element-wise 99.9th-percentile error beside it under a looser bar of its
own (it catches small entries that are wrong by a large factor, which the
norm-wise figure scales away)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import max_rel_err, rel_err_p999

TOL = {"f32": 1e-4, "bf16": 2e-2}
# bars of the element-wise figure, by the norm-wise bar they go with
P999_TOL = {1e-4: 5e-2, 2e-2: 5e-1}


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
    p999 = rel_err_p999(o, ref)
    ptol = P999_TOL.get(tol, 25.0 * tol)
    msg = (f"{name}: max_rel_err={err:.3e} (tol {tol:.1e}) "
           f"p999={p999:.3e} (tol {ptol:.1e})")
    print(msg, flush=True)
    if log is not None:
        log.append((name, err, p999))
    assert err <= tol, msg
    assert p999 <= ptol, msg
    return err
