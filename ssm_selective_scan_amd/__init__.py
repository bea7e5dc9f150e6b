"""Python binding of liblr — fused linear-recurrence scans on MI355X (gfx950).

Argument marshalling only: every function takes torch tensors on the GPU,
checks dtype/device/contiguity, allocates the outputs the caller did not
pass, and calls the C entry point of the same name (include/lr.h) on the
current torch stream.  All arithmetic happens in the HIP kernels of liblr.so;
there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import torch

from ._lib import (LR_BF16, LR_DISC_BILINEAR, LR_DISC_DIRAC, LR_DISC_EULER,  # noqa: F401
                   LR_DISC_ZOH, LR_F32, LrError, check, lib)

__all__ = ["lr_diag_scan", "lr_diag_scan_bwd", "lr_rotlru_scan", "lr_rotlru_scan_bwd", "lr_selective_scan", "lr_selective_scan_bwd",
           "lr_selective_scan_bwd_workspace_bytes", "lr_ssd_scan", "lr_ssd_scan_bwd",
           "lr_ssd_scan_bwd_workspace_bytes", "lr_gla_scan", "lr_gla_scan_bwd",
           "lr_gla_scan_bwd_workspace_bytes", "lr_diag_step", "lr_selective_step", "lr_ssd_step",
           "lr_gla_step", "lr_version", "LrError"]

_DISC = {"zoh": LR_DISC_ZOH, "euler": LR_DISC_EULER, "bilinear": LR_DISC_BILINEAR,
         "dirac": LR_DISC_DIRAC}


def _io(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LR_F32
    if t.dtype == torch.bfloat16:
        return LR_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() or None


def _f32(t, name):
    if t is not None and t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return _ptr(t)


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def lr_version() -> str:
    return lib().lr_version().decode()


def lr_diag_scan(a, b, h0=None, h=None, h_last=None, want_last=False):
    """h[b,t,d] = a[b,t,d] h[b,t-1,d] + b[b,t,d]; a, b: [B, L, D]."""
    B, L, D = a.shape
    if h is None:
        h = torch.empty_like(a)
    if want_last and h_last is None:
        h_last = torch.empty(B, D, device=a.device, dtype=torch.float32)
    check("lr_diag_scan", lib().lr_diag_scan(
        _io(a), B, L, D, _ptr(a), _ptr(b), _f32(h0, "h0"), _ptr(h), _f32(h_last, "h_last"),
        _stream(a)))
    return h, h_last


def lr_diag_scan_bwd(a, h, dh, h0=None, dh_last=None, want_dh0=False):
    """Gradients (da, db, dh0) of sum <dh, h> + <dh_last, h_last> through
    lr_diag_scan; h is the forward's output [B, L, D]."""
    B, L, D = a.shape
    da = torch.empty_like(a)
    db = torch.empty_like(a)
    dh0 = torch.empty(B, D, device=a.device, dtype=torch.float32) if want_dh0 else None
    check("lr_diag_scan_bwd", lib().lr_diag_scan_bwd(
        _io(a), B, L, D, _ptr(a), _ptr(h), _f32(h0, "h0"), _ptr(dh), _f32(dh_last, "dh_last"),
        _ptr(da), _ptr(db), _f32(dh0, "dh0"), _stream(a)))
    return da, db, dh0


def lr_rotlru_scan(r, theta, u, h0=None, h=None, h_last=None, want_last=False):
    """Rotational LRU; r, theta: [B, L, D/2]; u: [B, L, D] (interleaved pairs)."""
    B, L, D = u.shape
    if h is None:
        h = torch.empty_like(u)
    if want_last and h_last is None:
        h_last = torch.empty(B, D, device=u.device, dtype=torch.float32)
    check("lr_rotlru_scan", lib().lr_rotlru_scan(
        _io(u), B, L, D, _ptr(r), _ptr(theta), _ptr(u), _f32(h0, "h0"), _ptr(h),
        _f32(h_last, "h_last"), _stream(u)))
    return h, h_last



def lr_rotlru_scan_bwd(r, theta, h, dh, h0=None, dh_last=None, want_dh0=False):
    """Gradients (dr, dtheta, du, dh0) of sum <dh, h> + <dh_last, h_last>
    through lr_rotlru_scan; h is the forward's output [B, L, D]."""
    B, L, D = h.shape
    dr = torch.empty_like(r)
    dtheta = torch.empty_like(theta)
    du = torch.empty_like(h)
    dh0 = torch.empty(B, D, device=h.device, dtype=torch.float32) if want_dh0 else None
    check("lr_rotlru_scan_bwd", lib().lr_rotlru_scan_bwd(
        _io(h), B, L, D, _ptr(r), _ptr(theta), _ptr(h), _f32(h0, "h0"), _ptr(dh),
        _f32(dh_last, "dh_last"), _ptr(dr), _ptr(dtheta), _ptr(du), _f32(dh0, "dh0"), _stream(h)))
    return dr, dtheta, du, dh0

def lr_selective_scan(x, dt, A, Bm, Cm, Dskip=None, h0=None, disc="zoh", seg=0, y=None,
                      h_last=None, ckpt=None, want_last=False):
    """Mamba-1 selective scan with fused readout; x, dt: [B, L, D], A: [D, N],
    Bm, Cm: [B, L, N].  With seg > 0 the segment checkpoints
    ([ceil(L/seg), B, D, N]) are returned as the third value."""
    B, L, D = x.shape
    N = A.shape[1]
    if y is None:
        y = torch.empty_like(x)
    if want_last and h_last is None:
        h_last = torch.empty(B, D, N, device=x.device, dtype=torch.float32)
    if seg > 0 and ckpt is None:
        ckpt = torch.empty((L + seg - 1) // seg, B, D, N, device=x.device, dtype=torch.float32)
    check("lr_selective_scan", lib().lr_selective_scan(
        _io(x), _DISC[disc], B, L, D, N, seg, _ptr(x), _ptr(dt), _f32(A, "A"), _ptr(Bm),
        _ptr(Cm), _f32(Dskip, "Dskip"), _f32(h0, "h0"), _ptr(y), _f32(h_last, "h_last"),
        _f32(ckpt, "ckpt"), _stream(x)))
    return (y, h_last, ckpt) if seg > 0 else (y, h_last)


def lr_selective_scan_bwd_workspace_bytes(B, L, D, N, seg) -> int:
    return int(lib().lr_selective_scan_bwd_workspace_bytes(B, L, D, N, seg))


def lr_selective_scan_bwd(x, dt, A, Bm, Cm, Dskip, ckpt, dy, dh_last=None, disc="zoh", seg=256,
                          workspace=None, want_dh0=False):
    """Gradients of sum(dy*y) + <dh_last, h_last> of lr_selective_scan.
    Returns a dict with dx, ddt, dA, dB, dC, dD (None without Dskip), dh0."""
    B, L, D = x.shape
    N = A.shape[1]
    dev = x.device
    dx, ddt = torch.empty_like(x), torch.empty_like(dt)
    dB, dC = torch.empty_like(Bm), torch.empty_like(Cm)
    dA = torch.empty(D, N, device=dev, dtype=torch.float32)
    dD = torch.empty(D, device=dev, dtype=torch.float32) if Dskip is not None else None
    dh0 = torch.empty(B, D, N, device=dev, dtype=torch.float32) if want_dh0 else None
    need = lr_selective_scan_bwd_workspace_bytes(B, L, D, N, seg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
    check("lr_selective_scan_bwd", lib().lr_selective_scan_bwd(
        _io(x), _DISC[disc], B, L, D, N, seg, _ptr(x), _ptr(dt), _f32(A, "A"), _ptr(Bm),
        _ptr(Cm), _f32(Dskip, "Dskip"), _f32(ckpt, "ckpt"), _ptr(dy), _f32(dh_last, "dh_last"),
        _ptr(dx), _ptr(ddt), _f32(dA, "dA"), _ptr(dB), _ptr(dC), _f32(dD, "dD"),
        _f32(dh0, "dh0"), _ptr(workspace), workspace.numel(), _stream(x)))
    return dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD, dh0=dh0)


def _fwd_workspace(workspace, need, dev):
    """"auto": a fresh buffer of `need` bytes (None when no split is used);
    None: single pass; a uint8 tensor: used as given."""
    if isinstance(workspace, str):
        return torch.empty(need, device=dev, dtype=torch.uint8) if need > 0 else None
    return workspace


def lr_ssd_scan_workspace_bytes(B, L, H, P, G, N, chunk=64) -> int:
    return int(lib().lr_ssd_scan_workspace_bytes(B, L, H, P, G, N, chunk))


def lr_ssd_scan(x, dt, A, Bm, Cm, Dskip=None, h0=None, disc="zoh", chunk=64, seg=0, y=None,
                h_last=None, ckpt=None, want_last=False, workspace="auto"):
    """Mamba-2 SSD scan; x: [B, L, H, P], dt: [B, L, H], A: [H],
    Bm, Cm: [B, L, G, N].  With seg > 0 also returns the segment checkpoints.
    workspace: "auto", None (single pass) or a uint8 device tensor of at
    least lr_ssd_scan_workspace_bytes() bytes."""
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    ws = _fwd_workspace(workspace, lr_ssd_scan_workspace_bytes(B, L, H, P, G, N, chunk), x.device)
    if y is None:
        y = torch.empty_like(x)
    if want_last and h_last is None:
        h_last = torch.empty(B, H, P, N, device=x.device, dtype=torch.float32)
    if seg and ckpt is None:
        ckpt = torch.empty((L + seg - 1) // seg, B, H, P, N, device=x.device, dtype=torch.float32)
    check("lr_ssd_scan", lib().lr_ssd_scan(
        _io(x), _DISC[disc], B, L, H, P, G, N, chunk, seg, _ptr(x), _ptr(dt), _f32(A, "A"),
        _ptr(Bm), _ptr(Cm), _f32(Dskip, "Dskip"), _f32(h0, "h0"), _ptr(y),
        _f32(h_last, "h_last"), _f32(ckpt, "ckpt"), _ptr(ws), ws.numel() if ws is not None else 0,
        _stream(x)))
    return y, h_last, ckpt


def lr_ssd_scan_bwd_workspace_bytes(B, L, H, P, G, N, chunk, seg) -> int:
    return int(lib().lr_ssd_scan_bwd_workspace_bytes(B, L, H, P, G, N, chunk, seg))


def lr_ssd_scan_bwd(x, dt, A, Bm, Cm, Dskip, h0, ckpt, dy, dh_last=None, disc="zoh", chunk=64,
                    seg=64, workspace=None, want_dh0=False):
    """Gradients of sum(dy*y) + <dh_last, h_last> of lr_ssd_scan.  Returns a
    dict with dx, ddt, dA, dB, dC, dD (None without Dskip) and dh0."""
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dev = x.device
    dx, ddt = torch.empty_like(x), torch.empty_like(dt)
    dB, dC = torch.empty_like(Bm), torch.empty_like(Cm)
    dA = torch.empty(H, device=dev, dtype=torch.float32)
    dD = torch.empty(H, device=dev, dtype=torch.float32) if Dskip is not None else None
    dh0 = torch.empty(B, H, P, N, device=dev, dtype=torch.float32) if want_dh0 else None
    need = lr_ssd_scan_bwd_workspace_bytes(B, L, H, P, G, N, chunk, seg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
    check("lr_ssd_scan_bwd", lib().lr_ssd_scan_bwd(
        _io(x), _DISC[disc], B, L, H, P, G, N, chunk, seg, _ptr(x), _ptr(dt), _f32(A, "A"),
        _ptr(Bm), _ptr(Cm), _f32(Dskip, "Dskip"), _f32(h0, "h0"), _f32(ckpt, "ckpt"), _ptr(dy),
        _f32(dh_last, "dh_last"), _ptr(dx), _ptr(ddt), _f32(dA, "dA"), _ptr(dB), _ptr(dC),
        _f32(dD, "dD"), _f32(dh0, "dh0"), _ptr(workspace), workspace.numel(), _stream(x)))
    return dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD, dh0=dh0)


def lr_gla_scan_workspace_bytes(B, L, H, K, V, chunk=64) -> int:
    return int(lib().lr_gla_scan_workspace_bytes(B, L, H, K, V, chunk))


def lr_gla_scan(q, k, v, g, S0=None, chunk=64, seg=0, o=None, S_last=None, ckpt=None,
                want_last=False, workspace="auto"):
    """GLA; q, k: [B, L, H, K], v: [B, L, H, V], g: [B, L, H].  With seg > 0
    the segment checkpoints ([ceil(L/seg), B, H, V, K], the state transposed)
    are returned as the third value.  workspace: as in lr_ssd_scan."""
    B, L, H, K = q.shape
    V = v.shape[3]
    ws = _fwd_workspace(workspace, lr_gla_scan_workspace_bytes(B, L, H, K, V, chunk), q.device)
    if o is None:
        o = torch.empty_like(v)
    if want_last and S_last is None:
        S_last = torch.empty(B, H, K, V, device=q.device, dtype=torch.float32)
    if seg > 0 and ckpt is None:
        ckpt = torch.empty((L + seg - 1) // seg, B, H, V, K, device=q.device, dtype=torch.float32)
    check("lr_gla_scan", lib().lr_gla_scan(
        _io(q), B, L, H, K, V, chunk, seg, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _f32(S0, "S0"),
        _ptr(o), _f32(S_last, "S_last"), _f32(ckpt, "ckpt"), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(q)))
    return (o, S_last, ckpt) if seg > 0 else (o, S_last)


def lr_gla_scan_bwd_workspace_bytes(B, L, H, K, V, chunk, seg) -> int:
    return int(lib().lr_gla_scan_bwd_workspace_bytes(B, L, H, K, V, chunk, seg))


def lr_gla_scan_bwd(q, k, v, g, ckpt, dout, dS_last=None, chunk=64, seg=64, workspace=None,
                    want_dS0=False):
    """Gradients of sum(dout*o) + <dS_last, S_last> of lr_gla_scan.  Returns a
    dict with dq, dk, dv, dg and dS0."""
    B, L, H, K = q.shape
    V = v.shape[3]
    dev = q.device
    dq, dk, dv, dg = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g)
    dS0 = torch.empty(B, H, K, V, device=dev, dtype=torch.float32) if want_dS0 else None
    need = lr_gla_scan_bwd_workspace_bytes(B, L, H, K, V, chunk, seg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
    check("lr_gla_scan_bwd", lib().lr_gla_scan_bwd(
        _io(q), B, L, H, K, V, chunk, seg, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _f32(ckpt, "ckpt"),
        _ptr(dout), _f32(dS_last, "dS_last"), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
        _f32(dS0, "dS0"), _ptr(workspace), workspace.numel(), _stream(q)))
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dS0=dS0)


# ------------------------------------------------------------------ steps
def lr_diag_step(a, b, h, out=None):
    """h <- a h + b in place (h fp32 [B, D]); returns out = h in a's dtype."""
    B, D = a.shape
    if out is None:
        out = torch.empty_like(a)
    check("lr_diag_step", lib().lr_diag_step(_io(a), B, D, _ptr(a), _ptr(b), _f32(h, "h"),
                                             _ptr(out), _stream(a)))
    return out


def lr_selective_step(x, dt, A, Bm, Cm, Dskip, h, disc="zoh", y=None):
    """One token of lr_selective_scan; x, dt: [B, D]; Bm, Cm: [B, N]; h fp32
    [B, D, N] updated in place.  Returns y [B, D]."""
    B, D = x.shape
    N = A.shape[1]
    if y is None:
        y = torch.empty_like(x)
    check("lr_selective_step", lib().lr_selective_step(
        _io(x), _DISC[disc], B, D, N, _ptr(x), _ptr(dt), _f32(A, "A"), _ptr(Bm), _ptr(Cm),
        _f32(Dskip, "Dskip"), _f32(h, "h"), _ptr(y), _stream(x)))
    return y


def lr_ssd_step(x, dt, A, Bm, Cm, Dskip, h, disc="zoh", y=None):
    """One token of lr_ssd_scan; x: [B, H, P]; dt: [B, H]; Bm, Cm: [B, G, N];
    h fp32 [B, H, P, N] updated in place.  Returns y [B, H, P]."""
    B, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    if y is None:
        y = torch.empty_like(x)
    check("lr_ssd_step", lib().lr_ssd_step(
        _io(x), _DISC[disc], B, H, P, G, N, _ptr(x), _ptr(dt), _f32(A, "A"), _ptr(Bm), _ptr(Cm),
        _f32(Dskip, "Dskip"), _f32(h, "h"), _ptr(y), _stream(x)))
    return y


def lr_gla_step(q, k, v, g, S, o=None):
    """One token of lr_gla_scan; q, k: [B, H, K]; v: [B, H, V]; g: [B, H];
    S fp32 [B, H, K, V] updated in place.  Returns o [B, H, V]."""
    B, H, K = q.shape
    V = v.shape[2]
    if o is None:
        o = torch.empty_like(v)
    check("lr_gla_step", lib().lr_gla_step(_io(q), B, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                           _f32(S, "S"), _ptr(o), _stream(q)))
    return o
