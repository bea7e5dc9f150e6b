"""GPU parity of the selective-scan backward (segment checkpoints +
recompute) and of the forward's checkpoints against the fp64 oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import lrgen
import oracle
import ssm_selective_scan_amd as lr
from gpu_util import TOL, check, dev, host

pytestmark = pytest.mark.gpu


def _inputs(g, A=None):
    T = {k: dev(g.t(k)) for k in ("x", "dt", "B", "C", "dy")}
    T["A"] = dev(g["A"] if A is None else A, "f32")
    T["Dskip"] = dev(g.t("Dskip"))
    return T


def _fwd_bwd(T, seg, disc, h0=None, dhl=None):
    y, hl, ck = lr.lr_selective_scan(T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"],
                                     h0=None if h0 is None else dev(h0, "f32"), disc=disc, seg=seg,
                                     want_last=True)
    gr = lr.lr_selective_scan_bwd(T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"], ck, T["dy"],
                                  None if dhl is None else dev(dhl, "f32"), disc=disc, seg=seg,
                                  want_dh0=True)
    torch.cuda.synchronize()
    return ck, gr


@pytest.mark.parametrize("io,disc,B,L,D,N,seg,zero_A", [
    ("bf16", "zoh", 1, 64, 64, 16, 32, False),
    ("f32", "zoh", 2, 300, 70, 16, 64, False),
    ("bf16", "euler", 1, 513, 130, 5, 256, False),
    ("f32", "euler", 2, 65, 64, 8, 32, False),
    ("f32", "zoh", 1, 1, 3, 1, 32, False),
    ("f32", "zoh", 2, 200, 64, 16, 96, True),
    ("bf16", "zoh", 1, 777, 192, 12, 128, True),
    ("f32", "zoh", 2, 150, 70, 32, 32, False),
    ("bf16", "zoh", 1, 400, 64, 24, 256, False),
    ("f32", "euler", 1, 97, 130, 17, 96, False),
    ("f32", "zoh", 2, 260, 64, 32, 64, True),
    ("f32", "zoh", 1, 130, 70, 64, 32, False),
    ("bf16", "euler", 2, 300, 64, 40, 128, False),
    ("f32", "zoh", 1, 75, 66, 48, 64, True),
])
def test_selective_bwd_parity(io, disc, B, L, D, N, seg, zero_A):
    print(f"selective bwd io={io} disc={disc} B={B} L={L} D={D} N={N} seg={seg} zero_A={zero_A}",
          flush=True)
    g = lrgen.make(2, io=io, B=B, L=L, D=D, N=N, disc=disc, grads=True)
    A = g["A"].copy()
    if zero_A:
        A[::3] = 0.0
        A[1::3] *= 1e-3
    h0 = lrgen.state_normal((B, D, N), 2, tensor_id=21, std=0.5)
    dhl = lrgen.state_normal((B, D, N), 2, tensor_id=22, std=0.5)
    ck, gr = _fwd_bwd(_inputs(g, A), seg, disc, h0, dhl)
    ref = oracle.selective_scan_bwd(g["x"], g["dt"], A, g["B"], g["C"], g["Dskip"], h0, g["dy"], dhl,
                                    disc)
    for name in ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"):
        check(name, gr[name], ref[name], TOL[io])
    for s in range((L + seg - 1) // seg):
        if s == 0:
            st = h0
        else:
            _, st = oracle.selective_scan(g["x"][:, :s * seg], g["dt"][:, :s * seg], A,
                                          g["B"][:, :s * seg], g["C"][:, :s * seg], g["Dskip"], h0,
                                          disc)
        check(f"ckpt[{s}]", host(ck[s]), st, TOL["f32"] if io == "f32" else TOL["bf16"])


def test_selective_bwd_empty_and_determinism():
    dhl = torch.randn(2, 5, 4, device="cuda")
    z = torch.empty(2, 0, 5, device="cuda")
    zb = torch.empty(2, 0, 4, device="cuda")
    A = -torch.ones(5, 4, device="cuda")
    ck = torch.empty(0, 2, 5, 4, device="cuda")
    gr = lr.lr_selective_scan_bwd(z, z, A, zb, zb, torch.ones(5, device="cuda"), ck, z, dhl,
                                  seg=32, want_dh0=True)
    torch.cuda.synchronize()
    assert torch.equal(gr["dh0"], dhl)
    assert torch.count_nonzero(gr["dA"]) == 0 and torch.count_nonzero(gr["dD"]) == 0
    g = lrgen.make(2, B=2, L=300, D=130, grads=True)
    T = _inputs(g)
    _, g1 = _fwd_bwd(T, 64, "zoh")
    _, g2 = _fwd_bwd(T, 64, "zoh")
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"):
        assert torch.equal(g1[k], g2[k]), k


def test_selective_fwd_bwd_full_size_sampled():
    """B=8, L=4096, D=2048, N=16 (the Mamba-1 workload), seg=256: dD exactly;
    dx, ddt, dA of three channels over all batch rows; dB, dC, dx, ddt of the
    last 256 tokens of batch row 0 (state at the suffix start from an oracle
    prefix forward)."""
    print("selective fwd+bwd full size, sampled", flush=True)
    g = lrgen.make(2, grads=True)
    p = g.params
    B, L, D = p["B"], p["L"], p["D"]
    _, gr = _fwd_bwd(_inputs(g), 256, "zoh")
    ref_dD = np.einsum("bld,bld->d", g["dy"].astype(np.float64), g["x"].astype(np.float64))
    check("dD", gr["dD"], ref_dD, 1e-4)
    for d in (0, 777, 2047):
        c = slice(d, d + 1)
        r = oracle.selective_scan_bwd(g["x"][:, :, c], g["dt"][:, :, c], g["A"][c], g["B"], g["C"],
                                      g["Dskip"][c], None, g["dy"][:, :, c])
        check(f"dx[d={d}]", host(gr["dx"][:, :, c]), r["dx"], TOL["bf16"])
        check(f"ddt[d={d}]", host(gr["ddt"][:, :, c]), r["ddt"], TOL["bf16"])
        check(f"dA[d={d}]", host(gr["dA"][c]), r["dA"], TOL["bf16"])
    t0 = L - 256
    _, hpre = oracle.selective_scan(g["x"][:1, :t0], g["dt"][:1, :t0], g["A"], g["B"][:1, :t0],
                                    g["C"][:1, :t0], g["Dskip"])
    sfx = (slice(0, 1), slice(t0, L))
    r = oracle.selective_scan_bwd(g["x"][sfx], g["dt"][sfx], g["A"], g["B"][sfx], g["C"][sfx],
                                  g["Dskip"], hpre, g["dy"][sfx])
    for k in ("dB", "dC", "dx", "ddt"):
        check(f"{k}[b=0, last 256]", host(gr[k][sfx]), r[k], TOL["bf16"])
