"""Helpers for the GPU parity tests: upload seeded inputs, compare with the
oracle under the norm-wise max relative error bar."""
from __future__ import annotations

import numpy as np
import torch

from oracle import max_rel_err

TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev(t, io=None):
    """numpy float32 (bf16-representable when io == 'bf16') -> cuda tensor."""
    arr = t.values if hasattr(t, "values") else t
    io = io or (t.io if hasattr(t, "io") else "f32")
    x = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    return x.to(torch.bfloat16) if io == "bf16" else x


def host(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def check(name, out, ref, tol, log=None):
    err = max_rel_err(host(out) if torch.is_tensor(out) else out, ref)
    msg = f"{name}: max_rel_err={err:.3e} (tol {tol:.1e})"
    print(msg, flush=True)
    if log is not None:
        log.append((name, err))
    assert err <= tol, msg
    return err
