"""Boundary tests that run without a GPU: liblr.so loads, exports every
symbol declared in include/lr.h, and rejects invalid arguments with the
documented status code before touching the device (fake, never-dereferenced
pointer values are used; validation happens before any HIP call)."""
import ctypes as C

import pytest

from ssm_selective_scan_amd import _lib

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, OVF = 0, 1, 2, 3, 4, 5, 6, 7
P = 0x10000      # a fake 16-byte-aligned device address (never dereferenced)
MIS = 0x10008    # a fake misaligned one


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _lib.header_symbols()
    assert len(names) == len(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_version_and_status_strings(L):
    assert L.lr_version().decode().startswith("liblr")
    for code in range(9):
        assert L.lr_status_string(code).decode().startswith(_lib.STATUS[code])


def diag(L, io=0, B=1, Lq=8, D=4, a=P, b=P, h0=None, h=P, hl=None):
    return L.lr_diag_scan(io, B, Lq, D, a, b, h0, h, hl, None)


def test_diag_validation(L):
    assert diag(L, io=2) == DTYPE
    assert diag(L, D=0) == SHAPE
    assert diag(L, B=-1) == SHAPE
    assert diag(L, a=None) == NULL
    assert diag(L, h=None) == NULL
    assert diag(L, b=MIS) == ALIGN
    assert diag(L, h0=MIS) == ALIGN
    assert diag(L, B=1 << 40, Lq=1 << 20, D=1 << 10) == OVF
    # empty batch: nothing to do, no device access
    assert diag(L, B=0, a=None, b=None, h=None) == OK


def diag_bwd(L, io=0, B=1, Lq=8, D=4, a=P, h=P, h0=None, dh=P, dhl=None, da=P, db=P, dh0=None):
    return L.lr_diag_scan_bwd(io, B, Lq, D, a, h, h0, dh, dhl, da, db, dh0, None)


def test_diag_bwd_validation(L):
    assert diag_bwd(L, io=5) == DTYPE
    assert diag_bwd(L, D=0) == SHAPE
    assert diag_bwd(L, Lq=-1) == SHAPE
    for k in ("a", "h", "dh", "da", "db"):
        assert diag_bwd(L, **{k: None}) == NULL, k
    assert diag_bwd(L, dhl=MIS) == ALIGN
    assert diag_bwd(L, dh0=MIS) == ALIGN
    assert diag_bwd(L, B=1 << 40, Lq=1 << 20, D=1 << 10) == OVF
    assert diag_bwd(L, B=0, a=None, h=None, dh=None, da=None, db=None) == OK


def sel(L, io=1, disc=0, B=1, Lq=8, D=4, N=16, x=P, dt=P, A=P, Bm=P, Cm=P, y=P, seg=0, ck=None):
    return L.lr_selective_scan(io, disc, B, Lq, D, N, seg, x, dt, A, Bm, Cm, None, None, y, None, ck,
                               None)


def test_selective_ckpt_and_bwd_validation(L):
    assert sel(L, seg=48, ck=P) == UNSUP
    assert sel(L, seg=-32) == SHAPE
    assert sel(L, seg=32) == NULL        # checkpoints requested without a buffer
    assert sel(L, seg=32, ck=MIS) == ALIGN
    ws = L.lr_selective_scan_bwd_workspace_bytes(2, 100, 70, 16, 64)
    assert ws > 0
    assert L.lr_selective_scan_bwd_workspace_bytes(2, 100, 70, 65, 64) == 0
    assert L.lr_selective_scan_bwd_workspace_bytes(2, 100, 70, 16, 48) == 0
    #       io disc B  L    D   N   seg x  dt A  Bm Cm Dk    ckpt dy dhl   dx ddt dA dB dC dD    dh0
    args = [1, 0, 2, 100, 70, 16, 64, P, P, P, P, P, None, P, P, None, P, P, P, P, P, None, None]
    bad = list(args)
    bad[1] = 9
    assert L.lr_selective_scan_bwd(*bad, P, ws, None) == DTYPE
    bad = list(args)
    bad[6] = 0
    assert L.lr_selective_scan_bwd(*bad, P, ws, None) == SHAPE
    bad = list(args)
    bad[5] = 65
    assert L.lr_selective_scan_bwd(*bad, P, ws, None) == UNSUP
    bad = list(args)
    bad[13] = None   # ckpt
    assert L.lr_selective_scan_bwd(*bad, P, ws, None) == NULL
    bad = list(args)
    bad[18] = None   # dA
    assert L.lr_selective_scan_bwd(*bad, P, ws, None) == NULL
    bad = list(args)
    bad[16] = MIS    # dx
    assert L.lr_selective_scan_bwd(*bad, P, ws, None) == ALIGN
    assert L.lr_selective_scan_bwd(*args, P, ws - 256, None) == WS


def test_selective_validation(L):
    assert sel(L, disc=7) == DTYPE
    assert sel(L, disc=4) == DTYPE
    assert sel(L, N=0) == SHAPE
    assert sel(L, N=65) == UNSUP
    assert sel(L, A=None) == NULL
    assert sel(L, Cm=None) == NULL
    assert sel(L, dt=MIS) == ALIGN
    assert sel(L, B=0, x=None, dt=None, Bm=None, Cm=None, y=None) == OK
    assert sel(L, B=1, Lq=1, D=(1 << 24) + 1) == UNSUP   # 32-bit tile offsets
    assert sel(L, B=1 << 37, Lq=1, D=1 << 10, N=1) == OVF  # grid of 32-channel workgroups


def ssd(L, io=1, disc=0, B=1, Lq=64, H=2, Pp=64, G=1, N=128, chunk=64, seg=0, x=P, ck=None,
        ws=None, wsb=0):
    return L.lr_ssd_scan(io, disc, B, Lq, H, Pp, G, N, chunk, seg, x, P, P, P, P, None, None, P,
                         None, ck, ws, wsb, None)


def test_ssd_validation(L):
    assert ssd(L, io=0) == UNSUP          # fp32 I/O is not compiled for SSD
    assert ssd(L, H=3, G=2) == SHAPE
    assert ssd(L, Pp=48) == UNSUP
    assert ssd(L, N=96) == UNSUP
    assert ssd(L, chunk=100) == UNSUP
    assert ssd(L, seg=64) == NULL         # seg > 0 needs ckpt
    assert ssd(L, seg=96, ck=P) == UNSUP
    assert ssd(L, x=None) == NULL
    assert ssd(L, x=MIS) == ALIGN
    assert ssd(L, B=0, x=None) == OK
    # segments must be whole chunks
    assert ssd(L, chunk=256, seg=128, ck=P) == SHAPE
    assert ssd(L, chunk=128, seg=256, ck=P, x=None) == NULL


def test_ssd_row_width_limit(L):
    # 64 token rows of x (H*P elements) and of B/C (G*N) must stay within
    # 32-bit byte offsets: up to 2^25 elements per row.  At the limit the
    # sizes pass and the call stops at the missing pointer.
    assert ssd(L, H=1 << 19, x=None) == NULL            # H*P = 2^25
    assert ssd(L, H=(1 << 19) + 1, x=None) == UNSUP     # H*P = 2^25 + 64
    assert ssd(L, H=1 << 18, G=1 << 18, x=None) == NULL   # G*N = 2^25
    assert ssd(L, H=(1 << 18) + 1, G=(1 << 18) + 1, x=None) == UNSUP
    assert L.lr_ssd_scan_bwd_workspace_bytes(1, 64, (1 << 19) + 1, 64, 1, 128, 64, 64) == 0


def test_ssd_fwd_workspace(L):
    # few (batch, head) pairs and a long sequence: the forward splits the sequence
    need = L.lr_ssd_scan_workspace_bytes(1, 4096, 2, 64, 1, 128, 64)
    assert need > 0
    assert ssd(L, Lq=4096, ws=P, wsb=need - 1) == WS
    assert ssd(L, Lq=4096, ws=MIS, wsb=need) == ALIGN
    assert ssd(L, Lq=4096, x=None, ws=P, wsb=need) == NULL
    # enough workgroups already, or too short to split: no workspace
    assert L.lr_ssd_scan_workspace_bytes(8, 4096, 64, 64, 1, 128, 64) == 0
    assert L.lr_ssd_scan_workspace_bytes(1, 256, 2, 64, 1, 128, 64) == 0
    # the split starts below 256 workgroups of (batch, head, 64 columns of P):
    # 256 (B=8, H=32, P=64; GLA B=8, H=16, V=128) run in one pass, 255 split
    # (into ceil(512 / 255) = 3 parts, each part's end state and decay kept)
    assert L.lr_ssd_scan_workspace_bytes(8, 2048, 32, 64, 1, 128, 64) == 0
    assert L.lr_gla_scan_workspace_bytes(8, 4096, 16, 128, 128, 64) == 0
    need = L.lr_ssd_scan_workspace_bytes(5, 2048, 51, 64, 1, 128, 64)
    assert need >= 2 * 5 * 51 * 64 * 128 * 4 + 2 * 5 * 51 * 4
    assert L.lr_ssd_scan_workspace_bytes(1, 2048, 128, 128, 1, 128, 64) == 0   # 256 by P = 128
    # invalid sizes
    assert L.lr_ssd_scan_workspace_bytes(1, 4096, 2, 48, 1, 128, 64) == 0
    assert L.lr_gla_scan_workspace_bytes(1, 4096, 2, 128, 128, 64) > 0
    assert L.lr_gla_scan_workspace_bytes(1, 4096, 2, 32, 128, 64) == 0


def test_ssd_bwd_validation(L):
    ws = L.lr_ssd_scan_bwd_workspace_bytes(1, 64, 2, 64, 1, 128, 64, 64)
    args = [1, 0, 1, 64, 2, 64, 1, 128, 64, 64, P, P, P, P, P, None, None, P, P, None,
            P, P, P, P, P, None, None]
    if ws > 0:
        assert L.lr_ssd_scan_bwd(*args, None, 0, None) == WS
        assert L.lr_ssd_scan_bwd(*args, P, ws - 1, None) == WS
    bad = list(args)
    bad[1] = 9     # no such discretisation
    assert L.lr_ssd_scan_bwd(*bad, P, ws, None) == DTYPE
    bad = list(args)
    bad[9] = 0     # seg = 0
    assert L.lr_ssd_scan_bwd(*bad, P, ws, None) == SHAPE
    bad = list(args)
    bad[17] = None  # ckpt
    assert L.lr_ssd_scan_bwd(*bad, P, ws, None) == NULL


def test_gla_validation(L):
    def gla(io=1, K=128, V=128, chunk=64, seg=0, q=P, g=P, ck=None, ws=None, wsb=0, Lq=64):
        return L.lr_gla_scan(io, 1, Lq, 2, K, V, chunk, seg, q, P, P, g, None, P, None, ck, ws, wsb,
                             None)
    assert gla(io=3) == DTYPE
    assert gla(K=32) == UNSUP
    assert gla(V=96) == UNSUP
    assert gla(chunk=32) == UNSUP
    assert gla(seg=32, ck=P) == UNSUP
    assert gla(seg=-64) == SHAPE
    assert gla(q=None) == NULL
    assert gla(seg=64) == NULL          # checkpoints requested without a buffer
    assert gla(g=MIS) == ALIGN
    assert gla(seg=64, ck=MIS) == ALIGN
    need = L.lr_gla_scan_workspace_bytes(1, 4096, 2, 128, 128, 64)
    assert gla(Lq=4096, ws=P, wsb=need - 1) == WS
    assert gla(chunk=256, seg=128, ck=P) == SHAPE       # segments are whole chunks


def test_gla_row_width_limit(L):
    def gla(H, K, V, q=None):
        return L.lr_gla_scan(1, 1, 64, H, K, V, 64, 0, q, P, P, P, None, P, None, None, None, 0,
                             None)
    assert gla(1 << 18, 128, 64) == NULL                # H*K = 2^25
    assert gla((1 << 18) + 1, 128, 64) == UNSUP
    assert gla(1 << 18, 64, 128) == NULL                # H*V = 2^25
    assert gla(1 << 18, 64, 192) == UNSUP


def test_gla_bwd_validation(L):
    ws = L.lr_gla_scan_bwd_workspace_bytes(1, 64, 2, 128, 128, 64, 64)
    assert ws > 0
    assert L.lr_gla_scan_bwd_workspace_bytes(1, 64, 2, 128, 128, 64, 512) == 0
    #       io  B  L   H  K    V    chunk seg q  k  v  g  ckpt dout dSl  dq dk dv dg dS0
    args = [1, 1, 64, 2, 128, 128, 64, 64, P, P, P, P, P, P, None, P, P, P, P, None]
    bad = list(args)
    bad[0] = 7
    assert L.lr_gla_scan_bwd(*bad, P, ws, None) == DTYPE
    bad = list(args)
    bad[7] = 0      # seg = 0: no checkpoints to recompute from
    assert L.lr_gla_scan_bwd(*bad, P, ws, None) == SHAPE
    bad = list(args)
    bad[7] = 320    # seg beyond the compiled set
    assert L.lr_gla_scan_bwd(*bad, P, ws, None) == UNSUP
    bad = list(args)
    bad[12] = None  # ckpt
    assert L.lr_gla_scan_bwd(*bad, P, ws, None) == NULL
    bad = list(args)
    bad[18] = MIS   # dg
    assert L.lr_gla_scan_bwd(*bad, P, ws, None) == ALIGN
    assert L.lr_gla_scan_bwd(*args, P, ws - 256, None) == WS
    assert L.lr_gla_scan_bwd(*args, None, ws, None) == WS


def test_step_validation(L):
    assert L.lr_diag_step(4, 1, 8, P, P, P, None, None) == DTYPE
    assert L.lr_diag_step(0, 1, 0, P, P, P, None, None) == SHAPE
    assert L.lr_diag_step(0, 1, 8, P, None, P, None, None) == NULL
    assert L.lr_diag_step(0, 1, 8, P, P, MIS, None, None) == ALIGN
    assert L.lr_diag_step(0, 0, 8, None, None, None, None, None) == OK
    sel = lambda io=0, disc=0, N=16, h=P: L.lr_selective_step(io, disc, 1, 8, N, P, P, P, P, P,
                                                              None, h, P, None)
    assert sel(disc=5) == DTYPE
    assert sel(N=65) == UNSUP
    assert sel(h=None) == NULL
    assert sel(h=MIS) == ALIGN
    ssd = lambda io=1, N=128, G=1, H=4, h=P: L.lr_ssd_step(io, 0, 1, H, 64, G, N, P, P, P, P, P,
                                                           None, h, P, None)
    assert ssd(io=0) == UNSUP
    assert ssd(N=96) == UNSUP
    assert ssd(G=3) == SHAPE
    assert ssd(h=None) == NULL
    gla = lambda io=1, V=128, S=P: L.lr_gla_step(io, 1, 2, 128, V, P, P, P, P, S, P, None)
    assert gla(V=100) == UNSUP
    assert gla(io=0) == UNSUP
    assert gla(S=None) == NULL
    assert gla(S=MIS) == ALIGN


def test_rotlru_validation(L):
    rot = lambda io=0, B=1, D=8, r=P, th=P, u=P, h=P, h0=None: L.lr_rotlru_scan(
        io, B, 16, D, r, th, u, h0, h, None, None)
    assert rot(io=2) == DTYPE
    assert rot(D=7) == SHAPE
    assert rot(D=0) == SHAPE
    assert rot(th=None) == NULL
    assert rot(h=None) == NULL
    assert rot(u=MIS) == ALIGN
    assert rot(h0=MIS) == ALIGN
    assert rot(B=0, r=None, th=None, u=None, h=None) == OK


def test_rotlru_bwd_validation(L):
    rb = lambda io=0, B=1, D=8, r=P, th=P, h=P, dh=P, dr=P, dth=P, du=P, dh0=None: \
        L.lr_rotlru_scan_bwd(io, B, 16, D, r, th, h, None, dh, None, dr, dth, du, dh0, None)
    assert rb(io=2) == DTYPE
    assert rb(D=7) == SHAPE
    assert rb(D=0) == SHAPE
    assert rb(dth=None) == NULL
    assert rb(du=None) == NULL
    assert rb(h=MIS) == ALIGN
    assert rb(dh0=MIS) == ALIGN
    assert rb(B=0, r=None, th=None, h=None, dh=None, dr=None, dth=None, du=None) == OK


def test_bwd_workspace_batch_slices(L):
    # B=4, L=8192, H=32, P=64, N=128, seg 256: 1024 (head, segment) items per
    # batch row, so the backward runs one row at a time and its workspace holds
    # one row's partials plus the whole batch's dA/dD partials (4 KiB per row)
    full = L.lr_ssd_scan_bwd_workspace_bytes(4, 8192, 32, 64, 1, 128, 64, 256)
    one = L.lr_ssd_scan_bwd_workspace_bytes(1, 8192, 32, 64, 1, 128, 64, 256)
    assert full <= 200 * 2 ** 20
    assert full - one == 2 * 3 * 32 * 32 * 4
    gla = L.lr_gla_scan_bwd_workspace_bytes(8, 4096, 16, 128, 128, 64, 256)
    assert gla == (L.lr_gla_scan_bwd_workspace_bytes(2, 4096, 16, 128, 128, 64, 256)
                   + 2 * 6 * 32 * 16 * 4)
    # small problems fit in one slice: the workspace grows with B
    w1 = L.lr_ssd_scan_bwd_workspace_bytes(1, 200, 2, 64, 1, 128, 64, 64)
    w3 = L.lr_ssd_scan_bwd_workspace_bytes(3, 200, 2, 64, 1, 128, 64, 64)
    assert w3 > 2 * w1
    # below the one-row size the call is refused before any launch
    args = [1, 0, 3, 200, 2, 64, 1, 128, 64, 64, P, P, P, P, P, None, None, P, P, None,
            P, P, P, P, P, None, None]
    assert L.lr_ssd_scan_bwd(*args, P, w1 - 1, None) == WS
