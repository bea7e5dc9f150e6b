"""GPU parity of the forward scans against the fp64 oracle (same seeded
inputs, element by element), through the C ABI via the thin binding.

Small cases span several 64-token blocks and ragged tails; the full-size
workloads are checked on sampled channels / heads that the oracle computes
independently (every channel or head is an independent recurrence)."""
import numpy as np
import pytest
import torch

import lrgen
import oracle
import ssm_selective_scan_amd as lr
from gpu_util import TOL, check, dev, host

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ diag
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("B,L,D", [(1, 1, 1), (2, 65, 17), (1, 513, 5), (3, 1000, 33),
                                   (1, 2049, 16), (1, 1024, 256),
                                   # wide channel tiles: 4 and 2 channels per lane
                                   (64, 600, 512), (33, 130, 514), (40, 70, 1000)])
def test_diag_parity(io, B, L, D):
    print(f"diag io={io} B={B} L={L} D={D}", flush=True)
    g = lrgen.make(1, io=io, B=B, L=L, D=D)
    h0 = lrgen.state_normal((B, D), 1)
    h, hl = lr.lr_diag_scan(dev(g.t("a")), dev(g.t("b")), h0=dev(h0), want_last=True)
    _sync()
    ref, ref_last = oracle.diag_scan(g["a"], g["b"], h0)
    check("h", h, ref, TOL[io])
    check("h_last", hl, ref_last, TOL["f32"] if io == "f32" else TOL["bf16"])


def test_diag_empty_and_determinism():
    g = lrgen.make(1, B=2, L=0, D=7)
    h0 = torch.randn(2, 7, device="cuda")
    h, hl = lr.lr_diag_scan(torch.empty(2, 0, 7, device="cuda"), torch.empty(2, 0, 7, device="cuda"),
                            h0=h0, want_last=True)
    _sync()
    assert torch.equal(hl, h0)
    g = lrgen.make(1)
    a, b = dev(g.t("a")), dev(g.t("b"))
    r1, _ = lr.lr_diag_scan(a, b)
    r2, _ = lr.lr_diag_scan(a, b)
    _sync()
    assert torch.equal(r1, r2)


@pytest.mark.parametrize("D", [512, 514])
def test_diag_empty_sequence_wide_tiles(D):
    """L = 0 through the 4- and 2-channel-per-lane kernels (B * D large enough
    to select them): h_last is h0 for every channel, forward and backward."""
    B = 64
    h0 = torch.randn(B, D, device="cuda")
    z = torch.empty(B, 0, D, device="cuda")
    _, hl = lr.lr_diag_scan(z, z, h0=h0, want_last=True)
    _, _, dh0 = lr.lr_diag_scan_bwd(z, z, z, dh_last=h0, want_dh0=True)
    _sync()
    assert torch.equal(hl, h0) and torch.equal(dh0, h0)


# ------------------------------------------------------------- selective
def _sel_case(io, disc, B, L, D, N, zero_A=False, seed_cfg=2):
    g = lrgen.make(seed_cfg, io=io, B=B, L=L, D=D, N=N, disc=disc)
    A = g["A"].copy()
    if zero_A:
        A[::3] = 0.0
        A[1::3] *= 1e-3
    h0 = lrgen.state_normal((B, D, N), 2, std=0.5)
    args = dict(x=dev(g.t("x")), dt=dev(g.t("dt")), A=dev(A, "f32"), Bm=dev(g.t("B")),
                Cm=dev(g.t("C")), Dskip=dev(g.t("Dskip")), h0=dev(h0))
    y, hl = lr.lr_selective_scan(**args, disc=disc, want_last=True)
    _sync()
    ry, rl = oracle.selective_scan(g["x"], g["dt"], A, g["B"], g["C"], g["Dskip"], h0, disc)
    check("y", y, ry, TOL[io])
    check("h_last", hl, rl, TOL[io])


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
@pytest.mark.parametrize("B,L,D,N", [(1, 1, 1, 1), (2, 65, 33, 16), (1, 100, 70, 5),
                                     (2, 129, 64, 64), (1, 40, 20, 32), (3, 77, 200, 12),
                                     (2, 96, 128, 9)])
def test_selective_parity(io, disc, B, L, D, N):
    print(f"selective io={io} disc={disc} B={B} L={L} D={D} N={N}", flush=True)
    _sel_case(io, disc, B, L, D, N)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_selective_zero_and_tiny_A(io):
    print(f"selective A~0 io={io}", flush=True)
    _sel_case(io, "zoh", 2, 300, 40, 16, zero_A=True)


def test_selective_full_size_sampled():
    print("selective full size (B=8, L=4096, D=2048, N=16), sampled channels", flush=True)
    g = lrgen.make(2)
    y, hl = lr.lr_selective_scan(dev(g.t("x")), dev(g.t("dt")), dev(g.t("A")), dev(g.t("B")),
                                 dev(g.t("C")), dev(g.t("Dskip")), want_last=True)
    _sync()
    y2, _ = lr.lr_selective_scan(dev(g.t("x")), dev(g.t("dt")), dev(g.t("A")), dev(g.t("B")),
                                 dev(g.t("C")), dev(g.t("Dskip")))
    _sync()
    assert torch.equal(y, y2), "non-deterministic output"
    dsel = np.r_[0:64, 1000:1040, 1984:2048]
    for b in (0, 7):
        ry, rl = oracle.selective_scan(g["x"][b:b + 1, :, dsel], g["dt"][b:b + 1, :, dsel],
                                       g["A"][dsel], g["B"][b:b + 1], g["C"][b:b + 1],
                                       g["Dskip"][dsel])
        check(f"y[b={b}]", host(y[b:b + 1, :, dsel]), ry, TOL["bf16"])
        check(f"h_last[b={b}]", host(hl[b:b + 1, dsel]), rl, TOL["bf16"])



def test_selective_max_channels_sampled():
    """The largest channel count the entry point accepts (D = 2^24, 524288
    workgroups of the paired kernel) with a ragged 5-token sequence; sampled
    channels at both ends and in the middle against the oracle."""
    D = 1 << 24
    print(f"selective max D={D} B=1 L=5 N=16 bf16", flush=True)
    g = lrgen.make(2, B=1, L=5, D=D)
    y, hl = lr.lr_selective_scan(dev(g.t("x")), dev(g.t("dt")), dev(g.t("A")), dev(g.t("B")),
                                 dev(g.t("C")), dev(g.t("Dskip")), want_last=True)
    _sync()
    dsel = np.r_[0:40, D // 2 - 20:D // 2 + 20, D - 40:D]
    ry, rl = oracle.selective_scan(g["x"][:, :, dsel], g["dt"][:, :, dsel], g["A"][dsel], g["B"],
                                   g["C"], g["Dskip"][dsel])
    check("y", host(y[:, :, dsel]), ry, TOL["bf16"])
    check("h_last", host(hl[:, dsel]), rl, TOL["bf16"])

# -------------------------------------------------------------------- SSD
def _ssd(g, disc="zoh", h0=None, seg=0, chunk=64):
    return lr.lr_ssd_scan(dev(g.t("x")), dev(g.t("dt")), dev(g.t("A")), dev(g.t("B")),
                          dev(g.t("C")), dev(g.t("Dskip")), None if h0 is None else dev(h0),
                          disc=disc, chunk=chunk, seg=seg, want_last=True)


@pytest.mark.parametrize("disc", ["zoh", "euler"])
@pytest.mark.parametrize("B,L,H,G,N", [(1, 1, 1, 1, 128), (2, 63, 3, 1, 128), (1, 64, 2, 2, 64),
                                       (2, 65, 4, 2, 128), (1, 200, 2, 1, 64), (1, 257, 2, 1, 128)])
def test_ssd_parity(disc, B, L, H, G, N):
    print(f"ssd disc={disc} B={B} L={L} H={H} G={G} N={N}", flush=True)
    g = lrgen.make(3, B=B, L=L, H=H, G=G, N=N)
    h0 = lrgen.state_normal((B, H, 64, N), 3, std=0.3)
    seg = 64 if L > 1 else 0
    y, hl, ck = _ssd(g, disc, h0, seg=seg)
    _sync()
    ry, rl, rck = oracle.ssd_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], h0, disc,
                                  seg=seg)
    check("y", y, ry, TOL["bf16"])
    check("h_last", hl, rl, TOL["bf16"])
    if seg:
        check("ckpt", ck, rck, TOL["bf16"])


def test_ssd_chunk_invariance_and_determinism():
    g = lrgen.make(3, B=2, L=300, H=2)
    y64, h64, _ = _ssd(g, chunk=64)
    y256, h256, _ = _ssd(g, chunk=256)
    y64b, _, _ = _ssd(g, chunk=64)
    _sync()
    assert torch.equal(y64, y64b)
    assert torch.equal(y64, y256) and torch.equal(h64, h256)


@pytest.mark.parametrize("disc,L,seg,dt_scale,N,G", [("zoh", 1100, 128, 1.0, 128, 1),
                                                      ("euler", 2000, 64, 1.0, 64, 2),
                                                      ("bilinear", 1600, 192, 32.0, 128, 1),
                                                      ("dirac", 1031, 0, 1.0, 128, 1)])
def test_ssd_sequence_split(disc, L, seg, dt_scale, N, G):
    """Few (batch, head) pairs and a long sequence: the forward runs in parts
    (state-only pre-pass, then the fold of the parts' end states), including
    a ragged last part, checkpoints across part boundaries and, for bilinear,
    negative decays inside the parts' decay products."""
    B, H, P = 1, 2, 64
    print(f"ssd split disc={disc} L={L} seg={seg} dt_scale={dt_scale} N={N} G={G}", flush=True)
    assert lr.lr_ssd_scan_workspace_bytes(B, L, H, P, G, N) > 0
    g = lrgen.make(3, B=B, L=L, H=H, P=P, G=G, N=N)
    dt = lrgen.round_bf16(g["dt"] * dt_scale)
    h0 = lrgen.state_normal((B, H, P, N), 3, std=0.3)
    args = (dev(g.t("x")), dev(dt, "bf16"), dev(g.t("A")), dev(g.t("B")), dev(g.t("C")),
            dev(g.t("Dskip")), dev(h0, "f32"))
    y, hl, ck = lr.lr_ssd_scan(*args, disc=disc, seg=seg, want_last=True)
    y1, hl1, _ = lr.lr_ssd_scan(*args, disc=disc, seg=seg, want_last=True, workspace=None)
    _sync()
    ry, rl, rck = oracle.ssd_scan(g["x"], dt, g["A"], g["B"], g["C"], g["Dskip"], h0, disc,
                                  seg=seg)
    check("y", y, ry, TOL["bf16"])
    check("h_last", hl, rl, TOL["bf16"])
    if seg:
        check("ckpt", ck, rck, TOL["bf16"])
    check("y (single pass)", y1, ry, TOL["bf16"])
    check("h_last (single pass)", hl1, rl, TOL["bf16"])


def test_ssd_full_size_sampled():
    print("ssd full size (B=8, L=2048, H=32, P=64, N=128), sampled heads", flush=True)
    g = lrgen.make(3)
    y, hl, _ = _ssd(g, chunk=256)
    _sync()
    for b, hh in [(0, 0), (3, 17), (7, 31)]:
        ry, rl, _ = oracle.ssd_scan(g["x"][b:b + 1, :, hh:hh + 1], g["dt"][b:b + 1, :, hh:hh + 1],
                                    g["A"][hh:hh + 1], g["B"][b:b + 1], g["C"][b:b + 1],
                                    g["Dskip"][hh:hh + 1])
        check(f"y[b={b},h={hh}]", host(y[b:b + 1, :, hh:hh + 1]), ry, TOL["bf16"])
        check(f"h_last[b={b},h={hh}]", host(hl[b:b + 1, hh:hh + 1]), rl, TOL["bf16"])


# -------------------------------------------------------------------- GLA
@pytest.mark.parametrize("B,L,H,K,V", [(1, 1, 1, 128, 128), (2, 64, 2, 64, 64), (1, 100, 2, 128, 128),
                                       (2, 130, 1, 128, 64), (1, 257, 3, 64, 128),
                                       (1, 300, 2, 128, 256), (2, 70, 1, 64, 384)])
def test_gla_parity(B, L, H, K, V):
    print(f"gla B={B} L={L} H={H} K={K} V={V}", flush=True)
    g = lrgen.make(4, B=B, L=L, H=H, K=K, V=V)
    S0 = lrgen.state_normal((B, H, K, V), 4, std=0.3)
    o, Sl = lr.lr_gla_scan(dev(g.t("q")), dev(g.t("k")), dev(g.t("v")), dev(g.t("g")), S0=dev(S0),
                           want_last=True)
    _sync()
    ro, rS = oracle.gla_scan(g["q"], g["k"], g["v"], g["g"], S0)
    check("o", o, ro, TOL["bf16"])
    check("S_last", Sl, rS, TOL["bf16"])


def test_gla_sequence_split():
    """GLA with two 64-column slices of V, run in sequence parts, with S0 and
    checkpoints across part boundaries."""
    B, L, H, K, V, seg = 1, 1500, 2, 128, 128, 128
    print(f"gla split B={B} L={L} H={H} K={K} V={V} seg={seg}", flush=True)
    assert lr.lr_gla_scan_workspace_bytes(B, L, H, K, V) > 0
    g = lrgen.make(4, B=B, L=L, H=H, K=K, V=V)
    S0 = lrgen.state_normal((B, H, K, V), 4, std=0.3)
    o, Sl, ck = lr.lr_gla_scan(dev(g.t("q")), dev(g.t("k")), dev(g.t("v")), dev(g.t("g")),
                               S0=dev(S0), seg=seg, want_last=True)
    _sync()
    ro, rS = oracle.gla_scan(g["q"], g["k"], g["v"], g["g"], S0)
    check("o", o, ro, TOL["bf16"])
    check("S_last", Sl, rS, TOL["bf16"])
    for s_ in (0, 5, 11):
        _, st = oracle.gla_scan(g["q"][:, :s_ * seg], g["k"][:, :s_ * seg], g["v"][:, :s_ * seg],
                                g["g"][:, :s_ * seg], S0)
        check(f"ckpt[{s_}]", host(ck[s_]), np.swapaxes(st, -1, -2), TOL["bf16"])


def test_gla_full_size_sampled():
    print("gla full size (B=8, L=4096, H=16, K=V=128), sampled heads", flush=True)
    g = lrgen.make(4)
    o, Sl = lr.lr_gla_scan(dev(g.t("q")), dev(g.t("k")), dev(g.t("v")), dev(g.t("g")),
                           want_last=True)
    _sync()
    for b, hh in [(0, 0), (5, 9), (7, 15)]:
        sl = (slice(b, b + 1), slice(None), slice(hh, hh + 1))
        ro, rS = oracle.gla_scan(g["q"][sl], g["k"][sl], g["v"][sl], g["g"][sl])
        check(f"o[b={b},h={hh}]", host(o[sl]), ro, TOL["bf16"])
        check(f"S_last[b={b},h={hh}]", host(Sl[b:b + 1, hh:hh + 1]), rS, TOL["bf16"])
