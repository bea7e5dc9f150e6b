"""lr_ssd_scan_noalloc (the SSD forward whose sequence-split scratch is the
library's static device array) against lr_ssd_scan with a caller workspace,
through the C ABI: two calls in a row on shapes that split the sequence, the
second smaller than the first (the static array still holds the first
call's part states), each bit-identical to the workspace entry point and
within the bf16 bar of the fp64 oracle."""
import numpy as np
import pytest
import torch

import lrgen
import oracle
import ssm_selective_scan_amd as lr
from gpu_util import TOL, check, dev, host

pytestmark = pytest.mark.gpu

# (B, L, H, G, N, seg, oracle heads): the SSD fwd+bwd workload's shape, whose
# split takes 12.6 MB of scratch, then a short two-head sequence
CASES = [(4, 8192, 32, 1, 128, 256, [(0, 3), (3, 30)]),
         (1, 1100, 2, 2, 64, 128, None)]


def _run(B, L, H, G, N, seg, heads):
    P = 64
    need = lr.lr_ssd_scan_workspace_bytes(B, L, H, P, G, N)
    print(f"noalloc ssd B={B} L={L} H={H} G={G} N={N} seg={seg}: split scratch {need} bytes",
          flush=True)
    assert need > 0, "the shape must split the sequence"
    g = lrgen.make(5, B=B, L=L, H=H, G=G, N=N, seg=seg)
    h0 = lrgen.state_normal((B, H, P, N), 5, tensor_id=21, std=0.3)
    T = {k: dev(g.t(k)) for k in ("x", "dt", "A", "B", "C", "Dskip")}
    args = (T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"], dev(h0, "f32"))
    y1, hl1, ck1 = lr.lr_ssd_scan(*args, seg=seg, want_last=True)
    nseg = (L + seg - 1) // seg
    y2 = torch.empty_like(y1)
    hl2 = torch.empty_like(hl1)
    ck2 = torch.empty(nseg, B, H, P, N, device="cuda")
    lr.lr_ssd_scan_noalloc(*args, seg=seg, y=y2, h_last=hl2, ckpt=ck2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "y differs from lr_ssd_scan"
    assert torch.equal(hl1, hl2), "h_last differs from lr_ssd_scan"
    assert torch.equal(ck1, ck2), "checkpoints differ from lr_ssd_scan"
    if heads is None:
        ry, rl, rck = oracle.ssd_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], h0,
                                      seg=seg)
        check("y", y2, ry, TOL["bf16"])
        check("h_last", hl2, rl, TOL["bf16"])
        check("ckpt", ck2, rck, TOL["bf16"])
    else:
        for b, hh in heads:
            grp = hh // (H // G)
            sl = (slice(b, b + 1), slice(None), slice(hh, hh + 1))
            gs = (slice(b, b + 1), slice(None), slice(grp, grp + 1))
            ry, rl, _ = oracle.ssd_scan(g["x"][sl], g["dt"][sl], g["A"][hh:hh + 1], g["B"][gs],
                                        g["C"][gs], g["Dskip"][hh:hh + 1], h0[b:b + 1, hh:hh + 1])
            check(f"y[b={b},h={hh}]", host(y2[sl]), ry, TOL["bf16"])
            check(f"h_last[b={b},h={hh}]", host(hl2[b:b + 1, hh:hh + 1]), rl, TOL["bf16"])


def test_noalloc_matches_workspace_entry_point():
    for case in CASES:
        _run(*case)


def test_noalloc_without_split():
    # enough (batch, head) pairs to fill the GPU: no scratch used at all
    B, L, H, G, N = 8, 300, 64, 1, 128
    assert lr.lr_ssd_scan_workspace_bytes(B, L, H, 64, G, N) == 0
    g = lrgen.make(3, B=B, L=L, H=H, G=G, N=N)
    T = {k: dev(g.t(k)) for k in ("x", "dt", "A", "B", "C", "Dskip")}
    args = (T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"])
    y1, _, _ = lr.lr_ssd_scan(*args)
    y2, _, _ = lr.lr_ssd_scan_noalloc(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
