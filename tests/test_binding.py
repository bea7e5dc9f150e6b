"""The Python binding rejects mismatched arguments before any launch (CPU
only: the checks run on shapes, dtypes and devices; a call whose arguments
all match fails afterwards because the tensors are not on a GPU)."""
import pytest
import torch

import ssm_selective_scan_amd as lr

bf, f32 = torch.bfloat16, torch.float32


def z(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def _raises(match, fn, *a, **k):
    with pytest.raises((ValueError, TypeError), match=match):
        fn(*a, **k)


def _not_on_gpu(fn, *a, **k):
    with pytest.raises(ValueError, match="GPU"):
        fn(*a, **k)


# ------------------------------------------------------------------ SSD
B, L, H, P, G, N = 2, 130, 3, 64, 1, 128


def ssd_args():
    return dict(x=z(B, L, H, P), dt=z(B, L, H), A=z(H, dtype=f32), Bm=z(B, L, G, N),
                Cm=z(B, L, G, N), Dskip=z(H, dtype=f32))


def test_ssd_bwd_ckpt_of_another_segment_length():
    a = ssd_args()
    ck256 = z(1, B, H, P, N, dtype=f32)          # written with seg = 256
    dy = z(B, L, H, P)
    _raises("ckpt", lr.lr_ssd_scan_bwd, **a, h0=None, ckpt=ck256, dy=dy, seg=64)
    _raises("seg is required", lr.lr_ssd_scan_bwd, **a, h0=None, ckpt=ck256, dy=dy)
    _raises("seg must be > 0", lr.lr_ssd_scan_bwd, **a, h0=None, ckpt=ck256, dy=dy, seg=0)
    _not_on_gpu(lr.lr_ssd_scan_bwd, **a, h0=None, ckpt=ck256, dy=dy, seg=256)


def test_ssd_mismatched_inputs():
    a = ssd_args()
    for name, bad in [("dt", z(B, L, H + 1)), ("A", z(H, dtype=bf)), ("Bm", z(B, L - 1, G, N)),
                      ("Cm", z(B, L - 1, G, N)), ("Dskip", z(H + 1, dtype=f32)),
                      ("dt", z(B, L, H, dtype=f32))]:
        _raises(name, lr.lr_ssd_scan, **{**a, name: bad})
    _raises("h0", lr.lr_ssd_scan, **a, h0=z(B, H, N, P, dtype=f32))
    _raises("y", lr.lr_ssd_scan, **a, y=z(B, L, H, P, dtype=f32))
    _raises("ckpt", lr.lr_ssd_scan, **a, seg=64, ckpt=z(2, B, H, P, N, dtype=f32))
    _raises("discretisation", lr.lr_ssd_scan, **a, disc="rk4")
    _raises("workspace", lr.lr_ssd_scan, **a, workspace=z(16, dtype=f32))
    _raises("dy", lr.lr_ssd_scan_bwd, **a, h0=None, ckpt=z(3, B, H, P, N, dtype=f32),
            dy=z(B, L, H, 32), seg=64)
    _raises("dh_last", lr.lr_ssd_scan_bwd, **a, h0=None, ckpt=z(3, B, H, P, N, dtype=f32),
            dy=z(B, L, H, P), dh_last=z(B, H, P, N), seg=64)
    _not_on_gpu(lr.lr_ssd_scan, **a, seg=64, ckpt=z(3, B, H, P, N, dtype=f32))


# ------------------------------------------------------------- selective
def test_selective_mismatched_inputs():
    Bs, Ls, D, Ns = 2, 100, 40, 16
    a = dict(x=z(Bs, Ls, D), dt=z(Bs, Ls, D), A=z(D, Ns, dtype=f32), Bm=z(Bs, Ls, Ns),
             Cm=z(Bs, Ls, Ns), Dskip=z(D, dtype=f32))
    _raises("dt", lr.lr_selective_scan, **{**a, "dt": z(Bs, Ls, D, dtype=f32)})
    _raises("A", lr.lr_selective_scan, **{**a, "A": z(D + 1, Ns, dtype=f32)})
    _raises("Bm", lr.lr_selective_scan, **{**a, "Bm": z(Bs, Ls, Ns + 1)})
    _raises("h0", lr.lr_selective_scan, **a, h0=z(Bs, D, Ns))
    ck = z(4, Bs, D, Ns, dtype=f32)              # seg = 32 for L = 100
    dy = z(Bs, Ls, D)
    _raises("ckpt", lr.lr_selective_scan_bwd, **a, ckpt=ck, dy=dy, seg=256)
    _raises("seg is required", lr.lr_selective_scan_bwd, **a, ckpt=ck, dy=dy)
    _raises("dy", lr.lr_selective_scan_bwd, **a, ckpt=ck, dy=z(Bs, Ls, D, dtype=f32), seg=32)
    _not_on_gpu(lr.lr_selective_scan_bwd, **a, ckpt=ck, dy=dy, seg=32)


# ------------------------------------------------------------------- GLA
def test_gla_mismatched_inputs():
    Bg, Lg, Hg, K, V = 1, 200, 2, 128, 64
    a = dict(q=z(Bg, Lg, Hg, K), k=z(Bg, Lg, Hg, K), v=z(Bg, Lg, Hg, V), g=z(Bg, Lg, Hg))
    _raises("k", lr.lr_gla_scan, **{**a, "k": z(Bg, Lg, Hg, 64)})
    _raises("g", lr.lr_gla_scan, **{**a, "g": z(Bg, Lg, Hg, 1)})
    _raises("S0", lr.lr_gla_scan, **a, S0=z(Bg, Hg, V, K, dtype=f32))
    ck = z(4, Bg, Hg, V, K, dtype=f32)          # seg = 64
    do = z(Bg, Lg, Hg, V)
    _raises("ckpt", lr.lr_gla_scan_bwd, **a, ckpt=ck, dout=do, seg=128)
    _raises("ckpt", lr.lr_gla_scan_bwd, **a, ckpt=z(4, Bg, Hg, K, V, dtype=f32), dout=do, seg=64)
    _raises("seg is required", lr.lr_gla_scan_bwd, **a, ckpt=ck, dout=do)
    _raises("dout", lr.lr_gla_scan_bwd, **a, ckpt=ck, dout=z(Bg, Lg, Hg, K), seg=64)
    _not_on_gpu(lr.lr_gla_scan_bwd, **a, ckpt=ck, dout=do, seg=64)


# ------------------------------------------------- diag, rotLRU and steps
def test_elementwise_and_step_mismatches():
    a = z(2, 50, 8, dtype=f32)
    _raises("b", lr.lr_diag_scan, a, z(2, 50, 8))
    _raises("h0", lr.lr_diag_scan, a, a, h0=z(2, 9, dtype=f32))
    _raises("dh", lr.lr_diag_scan_bwd, a, a, z(2, 49, 8, dtype=f32))
    _raises("even", lr.lr_rotlru_scan, z(2, 5, 3, dtype=f32), z(2, 5, 3, dtype=f32),
            z(2, 5, 7, dtype=f32))
    _raises("theta", lr.lr_rotlru_scan, z(2, 5, 4, dtype=f32), z(2, 5, 3, dtype=f32),
            z(2, 5, 8, dtype=f32))
    _raises("h", lr.lr_diag_step, z(2, 8), z(2, 8), z(2, 8))
    _raises("Bm", lr.lr_selective_step, z(2, 8), z(2, 8), z(8, 4, dtype=f32), z(2, 5), z(2, 4),
            None, z(2, 8, 4, dtype=f32))
    _raises("S", lr.lr_gla_step, z(2, 3, 64), z(2, 3, 64), z(2, 3, 64), z(2, 3),
            z(2, 3, 64, 64))
    _not_on_gpu(lr.lr_diag_scan, a, a)
