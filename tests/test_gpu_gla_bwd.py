"""GPU parity of the GLA backward (segment checkpoints + recompute) and of
the forward's checkpoints against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import lrgen
import oracle
import ssm_selective_scan_amd as lr
from gpu_util import TOL, check, dev, host

pytestmark = pytest.mark.gpu


def _fwd_bwd(g, seg, S0=None, dSl=None):
    T = {k: dev(g.t(k)) for k in ("q", "k", "v", "g", "do")}
    S0d = None if S0 is None else dev(S0, "f32")
    o, Sl, ck = lr.lr_gla_scan(T["q"], T["k"], T["v"], T["g"], S0=S0d, seg=seg, want_last=True)
    gr = lr.lr_gla_scan_bwd(T["q"], T["k"], T["v"], T["g"], ck, T["do"],
                            None if dSl is None else dev(dSl, "f32"), seg=seg, want_dS0=True)
    torch.cuda.synchronize()
    return o, ck, gr


@pytest.mark.parametrize("B,L,H,K,V,seg", [(1, 64, 1, 64, 64, 64), (2, 200, 2, 128, 128, 128),
                                           (1, 300, 1, 128, 192, 256), (2, 65, 1, 64, 128, 64),
                                           (1, 513, 2, 128, 64, 192), (1, 1, 1, 64, 64, 64)])
def test_gla_bwd_parity(B, L, H, K, V, seg):
    print(f"gla bwd B={B} L={L} H={H} K={K} V={V} seg={seg}", flush=True)
    g = lrgen.make(4, B=B, L=L, H=H, K=K, V=V, grads=True)
    S0 = lrgen.state_normal((B, H, K, V), 4, tensor_id=21, std=0.3)
    dSl = lrgen.state_normal((B, H, K, V), 4, tensor_id=22, std=0.3)
    _, ck, gr = _fwd_bwd(g, seg, S0, dSl)
    ref = oracle.gla_scan_bwd(g["q"], g["k"], g["v"], g["g"], S0, g["do"], dSl)
    for name in ("dq", "dk", "dv", "dg", "dS0"):
        check(name, gr[name], ref[name], TOL["bf16"])
    # checkpoints: the state entering token s*seg, stored transposed [V, K]
    for s in range((L + seg - 1) // seg):
        if s == 0:
            st = S0
        else:
            _, st = oracle.gla_scan(g["q"][:, :s * seg], g["k"][:, :s * seg], g["v"][:, :s * seg],
                                    g["g"][:, :s * seg], S0)
        check(f"ckpt[{s}]", host(ck[s]), np.swapaxes(st, 2, 3), TOL["bf16"])


def test_gla_bwd_empty_and_determinism():
    dSl = torch.randn(2, 1, 64, 64, device="cuda")
    z4 = torch.empty(2, 0, 1, 64, device="cuda", dtype=torch.bfloat16)
    z3 = torch.empty(2, 0, 1, device="cuda", dtype=torch.bfloat16)
    ck = torch.empty(0, 2, 1, 64, 64, device="cuda")
    gr = lr.lr_gla_scan_bwd(z4, z4, z4, z3, ck, z4, dSl, seg=64, want_dS0=True)
    torch.cuda.synchronize()
    assert torch.equal(gr["dS0"], dSl)
    g = lrgen.make(4, B=2, L=300, H=2, grads=True)
    _, _, g1 = _fwd_bwd(g, 128)
    _, _, g2 = _fwd_bwd(g, 128)
    for k in ("dq", "dk", "dv", "dg", "dS0"):
        assert torch.equal(g1[k], g2[k]), k


def test_gla_fwd_bwd_full_size_sampled():
    """B=8, L=4096, H=16, K=V=128, seg=256: every gradient of one (batch, head)
    over the whole sequence, and of the last 256 tokens of batch row 0 over
    all heads (state at the suffix start from an oracle prefix forward)."""
    print("gla fwd+bwd full size, sampled", flush=True)
    g = lrgen.make(4, grads=True)
    p = g.params
    B, L, H = p["B"], p["L"], p["H"]
    seg = 256
    _, _, gr = _fwd_bwd(g, seg)
    bb, hh = 5, 11
    sl = (slice(bb, bb + 1), slice(None), slice(hh, hh + 1))
    r = oracle.gla_scan_bwd(g["q"][sl], g["k"][sl], g["v"][sl], g["g"][sl], None, g["do"][sl])
    for name in ("dq", "dk", "dv", "dg"):
        check(f"{name}[b={bb},h={hh}]", host(gr[name][sl]), r[name], TOL["bf16"])
    t0 = L - 256
    _, Spre = oracle.gla_scan(g["q"][:1, :t0], g["k"][:1, :t0], g["v"][:1, :t0], g["g"][:1, :t0])
    sfx = (slice(0, 1), slice(t0, L))
    r = oracle.gla_scan_bwd(g["q"][sfx], g["k"][sfx], g["v"][sfx], g["g"][sfx], Spre, g["do"][sfx])
    for name in ("dq", "dk", "dv", "dg"):
        check(f"{name}[b=0, last 256]", host(gr[name][sfx]), r[name], TOL["bf16"])


def test_gla_bwd_batch_slices_bit_identical():
    """One-row batch slices (a workspace below the default size) give the
    one-pass gradients bit for bit."""
    B, L, H, K, V, seg = 3, 200, 2, 128, 128, 64
    print(f"gla bwd batch slices B={B} L={L} H={H} K={K} V={V}", flush=True)
    g = lrgen.make(4, B=B, L=L, H=H, K=K, V=V, grads=True)
    dSl = lrgen.state_normal((B, H, K, V), 4, tensor_id=22, std=0.3)
    T = {k: dev(g.t(k)) for k in ("q", "k", "v", "g", "do")}
    _, _, ck = lr.lr_gla_scan(T["q"], T["k"], T["v"], T["g"], seg=seg, want_last=True)
    args = (T["q"], T["k"], T["v"], T["g"], ck, T["do"], dev(dSl, "f32"))
    full = lr.lr_gla_scan_bwd(*args, seg=seg, want_dS0=True)
    nseg = (L + seg - 1) // seg
    small = (lr.lr_gla_scan_bwd_workspace_bytes(1, L, H, K, V, 64, seg)
             + 8 * (B - 1) * H * (V // 64) * nseg + 512)
    assert small < lr.lr_gla_scan_bwd_workspace_bytes(B, L, H, K, V, 64, seg)
    part = lr.lr_gla_scan_bwd(*args, seg=seg, want_dS0=True,
                              workspace=torch.empty(small, device="cuda", dtype=torch.uint8))
    torch.cuda.synchronize()
    for k in ("dq", "dk", "dv", "dg", "dS0"):
        assert torch.equal(full[k], part[k]), k
