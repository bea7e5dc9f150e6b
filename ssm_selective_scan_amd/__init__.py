"""Python binding of liblr — fused linear-recurrence scans on MI355X (gfx950).

Argument marshalling only: every function takes torch tensors on the GPU,
checks each tensor's shape, dtype and device against the primary input (so
no mismatched buffer, e.g. checkpoints of another segment length, reaches a
kernel), and contiguity, allocates the outputs the caller did not pass, and
calls the C entry point of the same name (include/lr.h) on the current torch
stream.  All arithmetic happens in the HIP kernels of liblr.so;
there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import torch

from ._lib import (LR_BF16, LR_DISC_BILINEAR, LR_DISC_DIRAC, LR_DISC_EULER,  # noqa: F401
                   LR_DISC_ZOH, LR_F32, LrError, check, lib)

__all__ = ["lr_diag_scan", "lr_diag_scan_bwd", "lr_rotlru_scan", "lr_rotlru_scan_bwd", "lr_selective_scan", "lr_selective_scan_bwd",
           "lr_selective_scan_bwd_workspace_bytes", "lr_ssd_scan", "lr_ssd_scan_noalloc", "lr_ssd_scan_bwd",
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


def _disc(disc) -> int:
    if disc not in _DISC:
        raise ValueError(f"unknown discretisation {disc!r}; use one of {sorted(_DISC)}")
    return _DISC[disc]


def _seg(seg, name="seg") -> int:
    if seg is None:
        raise ValueError(f"{name} is required: the checkpoint interval of the forward")
    seg = int(seg)
    if seg < 0:
        raise ValueError(f"{name} must be >= 0, got {seg}")
    return seg


def _nseg(L, seg):
    return (L + seg - 1) // seg


def _dims(name, t, ndim):
    if not torch.is_tensor(t):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _expect(ref, name, t, shape, dtype):
    """Check an argument against the primary input ``ref``: same device,
    exactly ``shape`` and ``dtype``.  None (an absent optional) passes."""
    if t is None:
        return
    if not torch.is_tensor(t):
        raise TypeError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {ref.device}")


def _expect_ws(ref, workspace):
    if workspace is None:
        return
    if not torch.is_tensor(workspace) or workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise TypeError("workspace must be a 1-D torch.uint8 tensor")
    if workspace.device != ref.device:
        raise ValueError(f"workspace is on {workspace.device}, the inputs on {ref.device}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() or None


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def lr_version() -> str:
    return lib().lr_version().decode()


F32 = torch.float32


def lr_diag_scan(a, b, h0=None, h=None, h_last=None, want_last=False):
    """h[b,t,d] = a[b,t,d] h[b,t-1,d] + b[b,t,d]; a, b: [B, L, D]."""
    B, L, D = _dims("a", a, 3)
    io = a.dtype
    _expect(a, "b", b, (B, L, D), io)
    _expect(a, "h0", h0, (B, D), F32)
    _expect(a, "h", h, (B, L, D), io)
    _expect(a, "h_last", h_last, (B, D), F32)
    if h is None:
        h = torch.empty_like(a)
    if want_last and h_last is None:
        h_last = torch.empty(B, D, device=a.device, dtype=F32)
    check("lr_diag_scan", lib().lr_diag_scan(
        _io(a), B, L, D, _ptr(a), _ptr(b), _ptr(h0), _ptr(h), _ptr(h_last), _stream(a)))
    return h, h_last


def lr_diag_scan_bwd(a, h, dh, h0=None, dh_last=None, want_dh0=False):
    """Gradients (da, db, dh0) of sum <dh, h> + <dh_last, h_last> through
    lr_diag_scan; h is the forward's output [B, L, D]."""
    B, L, D = _dims("a", a, 3)
    io = a.dtype
    _expect(a, "h", h, (B, L, D), io)
    _expect(a, "dh", dh, (B, L, D), io)
    _expect(a, "h0", h0, (B, D), F32)
    _expect(a, "dh_last", dh_last, (B, D), F32)
    da = torch.empty_like(a)
    db = torch.empty_like(a)
    dh0 = torch.empty(B, D, device=a.device, dtype=F32) if want_dh0 else None
    check("lr_diag_scan_bwd", lib().lr_diag_scan_bwd(
        _io(a), B, L, D, _ptr(a), _ptr(h), _ptr(h0), _ptr(dh), _ptr(dh_last),
        _ptr(da), _ptr(db), _ptr(dh0), _stream(a)))
    return da, db, dh0


def _rot_dims(u):
    B, L, D = _dims("u", u, 3)
    if D % 2 != 0:
        raise ValueError(f"the channel count must be even (interleaved pairs), got {D}")
    return B, L, D


def lr_rotlru_scan(r, theta, u, h0=None, h=None, h_last=None, want_last=False):
    """Rotational LRU; r, theta: [B, L, D/2]; u: [B, L, D] (interleaved pairs)."""
    B, L, D = _rot_dims(u)
    io = u.dtype
    _expect(u, "r", r, (B, L, D // 2), io)
    _expect(u, "theta", theta, (B, L, D // 2), io)
    _expect(u, "h0", h0, (B, D), F32)
    _expect(u, "h", h, (B, L, D), io)
    _expect(u, "h_last", h_last, (B, D), F32)
    if h is None:
        h = torch.empty_like(u)
    if want_last and h_last is None:
        h_last = torch.empty(B, D, device=u.device, dtype=F32)
    check("lr_rotlru_scan", lib().lr_rotlru_scan(
        _io(u), B, L, D, _ptr(r), _ptr(theta), _ptr(u), _ptr(h0), _ptr(h), _ptr(h_last),
        _stream(u)))
    return h, h_last


def lr_rotlru_scan_bwd(r, theta, h, dh, h0=None, dh_last=None, want_dh0=False):
    """Gradients (dr, dtheta, du, dh0) of sum <dh, h> + <dh_last, h_last>
    through lr_rotlru_scan; h is the forward's output [B, L, D]."""
    B, L, D = _rot_dims(h)
    io = h.dtype
    _expect(h, "r", r, (B, L, D // 2), io)
    _expect(h, "theta", theta, (B, L, D // 2), io)
    _expect(h, "dh", dh, (B, L, D), io)
    _expect(h, "h0", h0, (B, D), F32)
    _expect(h, "dh_last", dh_last, (B, D), F32)
    dr = torch.empty_like(r)
    dtheta = torch.empty_like(theta)
    du = torch.empty_like(h)
    dh0 = torch.empty(B, D, device=h.device, dtype=F32) if want_dh0 else None
    check("lr_rotlru_scan_bwd", lib().lr_rotlru_scan_bwd(
        _io(h), B, L, D, _ptr(r), _ptr(theta), _ptr(h), _ptr(h0), _ptr(dh), _ptr(dh_last),
        _ptr(dr), _ptr(dtheta), _ptr(du), _ptr(dh0), _stream(h)))
    return dr, dtheta, du, dh0


def _sel_check(x, dt, A, Bm, Cm, Dskip, h0):
    B, L, D = _dims("x", x, 3)
    _dims("A", A, 2)
    N = A.shape[1]
    io = x.dtype
    _expect(x, "dt", dt, (B, L, D), io)
    _expect(x, "A", A, (D, N), F32)
    _expect(x, "Bm", Bm, (B, L, N), io)
    _expect(x, "Cm", Cm, (B, L, N), io)
    _expect(x, "Dskip", Dskip, (D,), F32)
    _expect(x, "h0", h0, (B, D, N), F32)
    return B, L, D, N, io


def lr_selective_scan(x, dt, A, Bm, Cm, Dskip=None, h0=None, disc="zoh", seg=0, y=None,
                      h_last=None, ckpt=None, want_last=False):
    """Mamba-1 selective scan with fused readout; x, dt: [B, L, D], A: [D, N],
    Bm, Cm: [B, L, N].  With seg > 0 the segment checkpoints
    ([ceil(L/seg), B, D, N]) are returned as the third value."""
    B, L, D, N, io = _sel_check(x, dt, A, Bm, Cm, Dskip, h0)
    seg = _seg(seg)
    _expect(x, "y", y, (B, L, D), io)
    _expect(x, "h_last", h_last, (B, D, N), F32)
    if seg > 0:
        _expect(x, "ckpt", ckpt, (_nseg(L, seg), B, D, N), F32)
    if y is None:
        y = torch.empty_like(x)
    if want_last and h_last is None:
        h_last = torch.empty(B, D, N, device=x.device, dtype=F32)
    if seg > 0 and ckpt is None:
        ckpt = torch.empty(_nseg(L, seg), B, D, N, device=x.device, dtype=F32)
    check("lr_selective_scan", lib().lr_selective_scan(
        _io(x), _disc(disc), B, L, D, N, seg, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm),
        _ptr(Dskip), _ptr(h0), _ptr(y), _ptr(h_last), _ptr(ckpt if seg > 0 else None),
        _stream(x)))
    return (y, h_last, ckpt) if seg > 0 else (y, h_last)


def lr_selective_scan_bwd_workspace_bytes(B, L, D, N, seg) -> int:
    return int(lib().lr_selective_scan_bwd_workspace_bytes(B, L, D, N, seg))


def lr_selective_scan_bwd(x, dt, A, Bm, Cm, Dskip, ckpt, dy, dh_last=None, disc="zoh", seg=None,
                          workspace=None, want_dh0=False):
    """Gradients of sum(dy*y) + <dh_last, h_last> of lr_selective_scan.
    ``seg`` must be the forward's checkpoint interval (ckpt is
    [ceil(L/seg), B, D, N]).  Returns a dict with dx, ddt, dA, dB, dC, dD
    (None without Dskip), dh0."""
    B, L, D, N, io = _sel_check(x, dt, A, Bm, Cm, Dskip, None)
    seg = _seg(seg)
    if seg == 0:
        raise ValueError("seg must be > 0: the backward recomputes from segment checkpoints")
    _expect(x, "ckpt", ckpt, (_nseg(L, seg), B, D, N), F32)
    _expect(x, "dy", dy, (B, L, D), io)
    _expect(x, "dh_last", dh_last, (B, D, N), F32)
    _expect_ws(x, workspace)
    dev = x.device
    dx, ddt = torch.empty_like(x), torch.empty_like(dt)
    dB, dC = torch.empty_like(Bm), torch.empty_like(Cm)
    dA = torch.empty(D, N, device=dev, dtype=F32)
    dD = torch.empty(D, device=dev, dtype=F32) if Dskip is not None else None
    dh0 = torch.empty(B, D, N, device=dev, dtype=F32) if want_dh0 else None
    need = lr_selective_scan_bwd_workspace_bytes(B, L, D, N, seg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
    check("lr_selective_scan_bwd", lib().lr_selective_scan_bwd(
        _io(x), _disc(disc), B, L, D, N, seg, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm),
        _ptr(Cm), _ptr(Dskip), _ptr(ckpt), _ptr(dy), _ptr(dh_last), _ptr(dx), _ptr(ddt),
        _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dD), _ptr(dh0), _ptr(workspace), workspace.numel(),
        _stream(x)))
    return dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD, dh0=dh0)


def _fwd_workspace(workspace, need, dev):
    """"auto": a fresh buffer of `need` bytes (None when no split is used);
    None: single pass; a uint8 tensor: used as given."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace must be 'auto', None or a uint8 tensor, got {workspace!r}")
        return torch.empty(need, device=dev, dtype=torch.uint8) if need > 0 else None
    return workspace


def _ssd_check(x, dt, A, Bm, Cm, Dskip, h0):
    B, L, H, P = _dims("x", x, 4)
    _, _, G, N = _dims("Bm", Bm, 4)
    io = x.dtype
    _expect(x, "dt", dt, (B, L, H), io)
    _expect(x, "A", A, (H,), F32)
    _expect(x, "Bm", Bm, (B, L, G, N), io)
    _expect(x, "Cm", Cm, (B, L, G, N), io)
    _expect(x, "Dskip", Dskip, (H,), F32)
    _expect(x, "h0", h0, (B, H, P, N), F32)
    return B, L, H, P, G, N, io


def lr_ssd_scan_workspace_bytes(B, L, H, P, G, N, chunk=64) -> int:
    return int(lib().lr_ssd_scan_workspace_bytes(B, L, H, P, G, N, chunk))


def lr_ssd_scan(x, dt, A, Bm, Cm, Dskip=None, h0=None, disc="zoh", chunk=64, seg=0, y=None,
                h_last=None, ckpt=None, want_last=False, workspace="auto"):
    """Mamba-2 SSD scan; x: [B, L, H, P], dt: [B, L, H], A: [H],
    Bm, Cm: [B, L, G, N].  With seg > 0 also returns the segment checkpoints.
    workspace: "auto", None (single pass) or a uint8 device tensor of at
    least lr_ssd_scan_workspace_bytes() bytes."""
    B, L, H, P, G, N, io = _ssd_check(x, dt, A, Bm, Cm, Dskip, h0)
    seg = _seg(seg)
    _expect(x, "y", y, (B, L, H, P), io)
    _expect(x, "h_last", h_last, (B, H, P, N), F32)
    if seg > 0:
        _expect(x, "ckpt", ckpt, (_nseg(L, seg), B, H, P, N), F32)
    ws = _fwd_workspace(workspace, lr_ssd_scan_workspace_bytes(B, L, H, P, G, N, chunk), x.device)
    _expect_ws(x, ws)
    if y is None:
        y = torch.empty_like(x)
    if want_last and h_last is None:
        h_last = torch.empty(B, H, P, N, device=x.device, dtype=F32)
    if seg > 0 and ckpt is None:
        ckpt = torch.empty(_nseg(L, seg), B, H, P, N, device=x.device, dtype=F32)
    check("lr_ssd_scan", lib().lr_ssd_scan(
        _io(x), _disc(disc), B, L, H, P, G, N, chunk, seg, _ptr(x), _ptr(dt), _ptr(A),
        _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(h0), _ptr(y), _ptr(h_last),
        _ptr(ckpt if seg > 0 else None), _ptr(ws), ws.numel() if ws is not None else 0,
        _stream(x)))
    return y, h_last, (ckpt if seg > 0 else None)


def lr_ssd_scan_noalloc(x, dt, A, Bm, Cm, Dskip=None, h0=None, disc="zoh", chunk=64, seg=0,
                        y=None, h_last=None, ckpt=None):
    """lr_ssd_scan whose sequence-split scratch is the library's static
    device array: the C call allocates nothing (pass y, h_last and ckpt to
    keep this wrapper from allocating them).  Returns (y, h_last, ckpt)."""
    B, L, H, P, G, N, io = _ssd_check(x, dt, A, Bm, Cm, Dskip, h0)
    seg = _seg(seg)
    _expect(x, "y", y, (B, L, H, P), io)
    _expect(x, "h_last", h_last, (B, H, P, N), F32)
    if seg > 0:
        _expect(x, "ckpt", ckpt, (_nseg(L, seg), B, H, P, N), F32)
    if y is None:
        y = torch.empty_like(x)
    if seg > 0 and ckpt is None:
        ckpt = torch.empty(_nseg(L, seg), B, H, P, N, device=x.device, dtype=F32)
    check("lr_ssd_scan_noalloc", lib().lr_ssd_scan_noalloc(
        _io(x), _disc(disc), B, L, H, P, G, N, chunk, seg, _ptr(x), _ptr(dt), _ptr(A),
        _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(h0), _ptr(y), _ptr(h_last),
        _ptr(ckpt if seg > 0 else None), _stream(x)))
    return y, h_last, (ckpt if seg > 0 else None)


def lr_ssd_scan_bwd_workspace_bytes(B, L, H, P, G, N, chunk, seg) -> int:
    return int(lib().lr_ssd_scan_bwd_workspace_bytes(B, L, H, P, G, N, chunk, seg))


def lr_ssd_scan_bwd(x, dt, A, Bm, Cm, Dskip, h0, ckpt, dy, dh_last=None, disc="zoh", chunk=64,
                    seg=None, workspace=None, want_dh0=False):
    """Gradients of sum(dy*y) + <dh_last, h_last> of lr_ssd_scan.  ``seg``
    must be the forward's checkpoint interval (ckpt is
    [ceil(L/seg), B, H, P, N]); h0, when given, is the forward's initial
    state.  Returns a dict with dx, ddt, dA, dB, dC, dD (None without
    Dskip) and dh0."""
    B, L, H, P, G, N, io = _ssd_check(x, dt, A, Bm, Cm, Dskip, h0)
    seg = _seg(seg)
    if seg == 0:
        raise ValueError("seg must be > 0: the backward recomputes from segment checkpoints")
    _expect(x, "ckpt", ckpt, (_nseg(L, seg), B, H, P, N), F32)
    _expect(x, "dy", dy, (B, L, H, P), io)
    _expect(x, "dh_last", dh_last, (B, H, P, N), F32)
    _expect_ws(x, workspace)
    dev = x.device
    dx, ddt = torch.empty_like(x), torch.empty_like(dt)
    dB, dC = torch.empty_like(Bm), torch.empty_like(Cm)
    dA = torch.empty(H, device=dev, dtype=F32)
    dD = torch.empty(H, device=dev, dtype=F32) if Dskip is not None else None
    dh0 = torch.empty(B, H, P, N, device=dev, dtype=F32) if want_dh0 else None
    need = lr_ssd_scan_bwd_workspace_bytes(B, L, H, P, G, N, chunk, seg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
    check("lr_ssd_scan_bwd", lib().lr_ssd_scan_bwd(
        _io(x), _disc(disc), B, L, H, P, G, N, chunk, seg, _ptr(x), _ptr(dt), _ptr(A),
        _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(h0), _ptr(ckpt), _ptr(dy), _ptr(dh_last),
        _ptr(dx), _ptr(ddt), _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dD), _ptr(dh0),
        _ptr(workspace), workspace.numel(), _stream(x)))
    return dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD, dh0=dh0)


def _gla_check(q, k, v, g):
    B, L, H, K = _dims("q", q, 4)
    V = _dims("v", v, 4)[3]
    io = q.dtype
    _expect(q, "k", k, (B, L, H, K), io)
    _expect(q, "v", v, (B, L, H, V), io)
    _expect(q, "g", g, (B, L, H), io)
    return B, L, H, K, V, io


def lr_gla_scan_workspace_bytes(B, L, H, K, V, chunk=64) -> int:
    return int(lib().lr_gla_scan_workspace_bytes(B, L, H, K, V, chunk))


def lr_gla_scan(q, k, v, g, S0=None, chunk=64, seg=0, o=None, S_last=None, ckpt=None,
                want_last=False, workspace="auto"):
    """GLA; q, k: [B, L, H, K], v: [B, L, H, V], g: [B, L, H].  With seg > 0
    the segment checkpoints ([ceil(L/seg), B, H, V, K], the state transposed)
    are returned as the third value.  workspace: as in lr_ssd_scan."""
    B, L, H, K, V, io = _gla_check(q, k, v, g)
    seg = _seg(seg)
    _expect(q, "S0", S0, (B, H, K, V), F32)
    _expect(q, "o", o, (B, L, H, V), io)
    _expect(q, "S_last", S_last, (B, H, K, V), F32)
    if seg > 0:
        _expect(q, "ckpt", ckpt, (_nseg(L, seg), B, H, V, K), F32)
    ws = _fwd_workspace(workspace, lr_gla_scan_workspace_bytes(B, L, H, K, V, chunk), q.device)
    _expect_ws(q, ws)
    if o is None:
        o = torch.empty_like(v)
    if want_last and S_last is None:
        S_last = torch.empty(B, H, K, V, device=q.device, dtype=F32)
    if seg > 0 and ckpt is None:
        ckpt = torch.empty(_nseg(L, seg), B, H, V, K, device=q.device, dtype=F32)
    check("lr_gla_scan", lib().lr_gla_scan(
        _io(q), B, L, H, K, V, chunk, seg, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0),
        _ptr(o), _ptr(S_last), _ptr(ckpt if seg > 0 else None), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(q)))
    return (o, S_last, ckpt) if seg > 0 else (o, S_last)


def lr_gla_scan_bwd_workspace_bytes(B, L, H, K, V, chunk, seg) -> int:
    return int(lib().lr_gla_scan_bwd_workspace_bytes(B, L, H, K, V, chunk, seg))


def lr_gla_scan_bwd(q, k, v, g, ckpt, dout, dS_last=None, chunk=64, seg=None, workspace=None,
                    want_dS0=False):
    """Gradients of sum(dout*o) + <dS_last, S_last> of lr_gla_scan.  ``seg``
    must be the forward's checkpoint interval (ckpt is
    [ceil(L/seg), B, H, V, K]).  Returns a dict with dq, dk, dv, dg and dS0."""
    B, L, H, K, V, io = _gla_check(q, k, v, g)
    seg = _seg(seg)
    if seg == 0:
        raise ValueError("seg must be > 0: the backward recomputes from segment checkpoints")
    _expect(q, "ckpt", ckpt, (_nseg(L, seg), B, H, V, K), F32)
    _expect(q, "dout", dout, (B, L, H, V), io)
    _expect(q, "dS_last", dS_last, (B, H, K, V), F32)
    _expect_ws(q, workspace)
    dev = q.device
    dq, dk, dv, dg = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g)
    dS0 = torch.empty(B, H, K, V, device=dev, dtype=F32) if want_dS0 else None
    need = lr_gla_scan_bwd_workspace_bytes(B, L, H, K, V, chunk, seg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
    check("lr_gla_scan_bwd", lib().lr_gla_scan_bwd(
        _io(q), B, L, H, K, V, chunk, seg, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(ckpt),
        _ptr(dout), _ptr(dS_last), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
        _ptr(dS0), _ptr(workspace), workspace.numel(), _stream(q)))
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dS0=dS0)


# ------------------------------------------------------------------ steps
def lr_diag_step(a, b, h, out=None):
    """h <- a h + b in place (h fp32 [B, D]); returns out = h in a's dtype."""
    B, D = _dims("a", a, 2)
    _expect(a, "b", b, (B, D), a.dtype)
    _expect(a, "h", h, (B, D), F32)
    _expect(a, "out", out, (B, D), a.dtype)
    if out is None:
        out = torch.empty_like(a)
    check("lr_diag_step", lib().lr_diag_step(_io(a), B, D, _ptr(a), _ptr(b), _ptr(h),
                                             _ptr(out), _stream(a)))
    return out


def lr_selective_step(x, dt, A, Bm, Cm, Dskip, h, disc="zoh", y=None):
    """One token of lr_selective_scan; x, dt: [B, D]; Bm, Cm: [B, N]; h fp32
    [B, D, N] updated in place.  Returns y [B, D]."""
    B, D = _dims("x", x, 2)
    _dims("A", A, 2)
    N = A.shape[1]
    io = x.dtype
    _expect(x, "dt", dt, (B, D), io)
    _expect(x, "A", A, (D, N), F32)
    _expect(x, "Bm", Bm, (B, N), io)
    _expect(x, "Cm", Cm, (B, N), io)
    _expect(x, "Dskip", Dskip, (D,), F32)
    _expect(x, "h", h, (B, D, N), F32)
    _expect(x, "y", y, (B, D), io)
    if y is None:
        y = torch.empty_like(x)
    check("lr_selective_step", lib().lr_selective_step(
        _io(x), _disc(disc), B, D, N, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm),
        _ptr(Dskip), _ptr(h), _ptr(y), _stream(x)))
    return y


def lr_ssd_step(x, dt, A, Bm, Cm, Dskip, h, disc="zoh", y=None):
    """One token of lr_ssd_scan; x: [B, H, P]; dt: [B, H]; Bm, Cm: [B, G, N];
    h fp32 [B, H, P, N] updated in place.  Returns y [B, H, P]."""
    B, H, P = _dims("x", x, 3)
    _, G, N = _dims("Bm", Bm, 3)
    io = x.dtype
    _expect(x, "dt", dt, (B, H), io)
    _expect(x, "A", A, (H,), F32)
    _expect(x, "Bm", Bm, (B, G, N), io)
    _expect(x, "Cm", Cm, (B, G, N), io)
    _expect(x, "Dskip", Dskip, (H,), F32)
    _expect(x, "h", h, (B, H, P, N), F32)
    _expect(x, "y", y, (B, H, P), io)
    if y is None:
        y = torch.empty_like(x)
    check("lr_ssd_step", lib().lr_ssd_step(
        _io(x), _disc(disc), B, H, P, G, N, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm),
        _ptr(Dskip), _ptr(h), _ptr(y), _stream(x)))
    return y


def lr_gla_step(q, k, v, g, S, o=None):
    """One token of lr_gla_scan; q, k: [B, H, K]; v: [B, H, V]; g: [B, H];
    S fp32 [B, H, K, V] updated in place.  Returns o [B, H, V]."""
    B, H, K = _dims("q", q, 3)
    V = _dims("v", v, 3)[2]
    io = q.dtype
    _expect(q, "k", k, (B, H, K), io)
    _expect(q, "v", v, (B, H, V), io)
    _expect(q, "g", g, (B, H), io)
    _expect(q, "S", S, (B, H, K, V), F32)
    _expect(q, "o", o, (B, H, V), io)
    if o is None:
        o = torch.empty_like(v)
    check("lr_gla_step", lib().lr_gla_step(_io(q), B, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                           _ptr(S), _ptr(o), _stream(q)))
    return o
