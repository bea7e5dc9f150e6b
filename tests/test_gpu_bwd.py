"""GPU parity of the SSD backward (segment checkpoints + recompute) against
the fp64 oracle's reverse-time adjoint, through the C ABI."""
import numpy as np
import pytest
import torch

import lrgen
import oracle
import ssm_selective_scan_amd as lr
from gpu_util import TOL, check, dev, host

pytestmark = pytest.mark.gpu


def _fwd_bwd(g, seg, disc="zoh", h0=None, dh_last=None):
    T = {k: dev(g.t(k)) for k in ("x", "dt", "A", "B", "C", "Dskip", "dy")}
    h0d = None if h0 is None else dev(h0, "f32")
    y, hl, ck = lr.lr_ssd_scan(T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"], h0d,
                               disc=disc, seg=seg, want_last=True)
    grads = lr.lr_ssd_scan_bwd(T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"], h0d, ck,
                               T["dy"], None if dh_last is None else dev(dh_last, "f32"),
                               disc=disc, seg=seg, want_dh0=True)
    torch.cuda.synchronize()
    return y, ck, grads


@pytest.mark.parametrize("disc", ["zoh", "euler"])
@pytest.mark.parametrize("B,L,H,G,N,seg", [(1, 64, 1, 1, 128, 64), (2, 200, 3, 1, 128, 128),
                                           (1, 300, 4, 2, 64, 256), (2, 65, 2, 1, 128, 64),
                                           (1, 513, 2, 1, 128, 192), (1, 1, 1, 1, 64, 64)])
def test_ssd_bwd_parity(disc, B, L, H, G, N, seg):
    print(f"ssd bwd disc={disc} B={B} L={L} H={H} G={G} N={N} seg={seg}", flush=True)
    g = lrgen.make(5, B=B, L=L, H=H, G=G, N=N, seg=seg)
    h0 = lrgen.state_normal((B, H, 64, N), 5, tensor_id=21, std=0.3)
    dhl = lrgen.state_normal((B, H, 64, N), 5, tensor_id=22, std=0.3)
    _, _, gr = _fwd_bwd(g, seg, disc, h0, dhl)
    ref = oracle.ssd_scan_bwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], h0, g["dy"],
                              dhl, disc)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"):
        check(k, gr[k], ref[k], TOL["bf16"])


def test_ssd_bwd_empty():
    x = torch.empty(2, 0, 2, 64, device="cuda", dtype=torch.bfloat16)
    dt = torch.empty(2, 0, 2, device="cuda", dtype=torch.bfloat16)
    Bm = torch.empty(2, 0, 1, 128, device="cuda", dtype=torch.bfloat16)
    A = torch.tensor([-1.0, -2.0], device="cuda")
    Dk = torch.ones(2, device="cuda")
    dhl = torch.randn(2, 2, 64, 128, device="cuda")
    gr = lr.lr_ssd_scan_bwd(x, dt, A, Bm, Bm, Dk, None, torch.empty(0, 2, 2, 64, 128, device="cuda"),
                            x, dhl, seg=64, want_dh0=True)
    torch.cuda.synchronize()
    assert torch.equal(gr["dh0"], dhl)
    assert torch.count_nonzero(gr["dA"]) == 0 and torch.count_nonzero(gr["dD"]) == 0


def test_ssd_bwd_determinism():
    g = lrgen.make(5, B=2, L=300, H=3, N=128, seg=128)
    _, _, g1 = _fwd_bwd(g, 128)
    _, _, g2 = _fwd_bwd(g, 128)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"):
        assert torch.equal(g1[k], g2[k]), k


def test_ssd_fwd_bwd_full_size_sampled():
    """B=4, L=8192, H=32, P=64, N=128, seg=256 (the checkpointed training
    workload): dD exactly, dx/ddt/dA on one head over all batch rows, and
    dB/dC/dx/ddt on the last 256 tokens of batch row 0 over all heads."""
    print("ssd fwd+bwd full size, sampled", flush=True)
    g = lrgen.make(5)
    p = g.params
    B, L, H, N, seg = p["B"], p["L"], p["H"], p["N"], p["seg"]
    y, ck, gr = _fwd_bwd(g, seg)
    assert ck.shape == ((L + seg - 1) // seg, B, H, 64, N)
    # dD[h] = sum <dy, x> exactly (no recurrence involved)
    ref_dD = np.einsum("blhp,blhp->h", g["dy"].astype(np.float64), g["x"].astype(np.float64))
    check("dD", gr["dD"], ref_dD, 1e-4)
    # one head, all batch rows: dx, ddt and dA[h]
    hh = 5
    dA = 0.0
    for b in range(B):
        sl = (slice(b, b + 1), slice(None), slice(hh, hh + 1))
        r = oracle.ssd_scan_bwd(g["x"][sl], g["dt"][sl], g["A"][hh:hh + 1], g["B"][b:b + 1],
                                g["C"][b:b + 1], g["Dskip"][hh:hh + 1], None, g["dy"][sl])
        check(f"dx[b={b},h={hh}]", host(gr["dx"][sl]), r["dx"], TOL["bf16"])
        check(f"ddt[b={b},h={hh}]", host(gr["ddt"][sl]), r["ddt"], TOL["bf16"])
        dA += r["dA"][0]
    check(f"dA[h={hh}]", host(gr["dA"][hh:hh + 1]), np.array([dA]), TOL["bf16"])
    # batch row 0, last 256 tokens, all heads: state at t0 from a prefix
    # forward, then the exact backward of the suffix
    t0 = L - 256
    _, hpre, _ = oracle.ssd_scan(g["x"][:1, :t0], g["dt"][:1, :t0], g["A"], g["B"][:1, :t0],
                                 g["C"][:1, :t0], g["Dskip"])
    sfx = (slice(0, 1), slice(t0, L))
    r = oracle.ssd_scan_bwd(g["x"][sfx], g["dt"][sfx], g["A"], g["B"][sfx], g["C"][sfx],
                            g["Dskip"], hpre, g["dy"][sfx])
    for k in ("dB", "dC", "dx", "ddt"):
        check(f"{k}[b=0, last 256]", host(gr[k][sfx]), r[k], TOL["bf16"])


def _inner(a, b):
    return float((a.double() * b.double()).sum())


def _noise_floor(a, b):
    # size of sum(a*b) if its terms had random signs: the scale against which
    # per-element rounding of a or b shows in the sum
    return float(((a.double() * b.double()) ** 2).sum().sqrt())


def test_ssd_fwd_bwd_full_size_linearity():
    """Whole tensors at B=4, L=8192, H=32, P=64, N=128, seg=256.  y is linear
    in x, so <dy, y(x=v)> = <dx, v> for any v (Dskip included); with h0 = 0,
    y - Dskip x is linear in B and in C, so <dy, y(B=w) - Dskip x> = <dB, w>
    and <dy, y(C=w) - Dskip x> = <dC, w>.  The gradients come from the
    backward at the workload's inputs, the left sides from forwards at v, w."""
    print("ssd fwd+bwd full size, linearity identities", flush=True)
    g = lrgen.make(5)
    p = g.params
    B, L, H, P, G, N, seg = p["B"], p["L"], p["H"], p["P"], p["G"], p["N"], p["seg"]
    _, _, gr = _fwd_bwd(g, seg)
    T = {k: dev(g.t(k)) for k in ("x", "dt", "A", "B", "C", "Dskip", "dy")}
    v = dev(lrgen.round_bf16(lrgen.state_normal((B, L, H, P), 5, tensor_id=31)), "bf16")
    w = dev(lrgen.round_bf16(lrgen.state_normal((B, L, G, N), 5, tensor_id=32)), "bf16")
    Dx = T["Dskip"].double()[None, None, :, None] * T["x"].double()
    fwd = lambda x, Bm, Cm: lr.lr_ssd_scan(x, T["dt"], T["A"], Bm, Cm, T["Dskip"],
                                           chunk=p["chunk"])[0]
    cases = [("x", fwd(v, T["B"], T["C"]).double(), gr["dx"], v),
             ("B", fwd(T["x"], w, T["C"]).double() - Dx, gr["dB"], w),
             ("C", fwd(T["x"], T["B"], w).double() - Dx, gr["dC"], w)]
    torch.cuda.synchronize()
    for name, yv, grad, probe in cases:
        lhs, rhs = _inner(T["dy"], yv), _inner(grad, probe)
        err = abs(lhs - rhs) / _noise_floor(T["dy"], yv)
        print(f"<dy, y({name}=probe)> = {lhs:.6e}, <d{name}, probe> = {rhs:.6e}, "
              f"|diff| / noise floor = {err:.3e}", flush=True)
        assert err <= TOL["bf16"], name


def _one_row_ws(B, L, H, P, G, N, seg):
    nseg = (L + seg - 1) // seg
    return lr.lr_ssd_scan_bwd_workspace_bytes(1, L, H, P, G, N, 64, seg) + 8 * (B - 1) * H * nseg + 512


@pytest.mark.parametrize("disc", ["zoh", "bilinear"])
def test_ssd_bwd_batch_slices_bit_identical(disc):
    """A workspace for one-row batch slices runs the backward slice by slice
    (one launch sequence per row); every gradient equals the one-pass result
    bit for bit, and (ZOH) the one-pass result matches the oracle."""
    B, L, H, G, N, seg = 3, 200, 2, 1, 128, 64
    print(f"ssd bwd batch slices disc={disc} B={B} L={L} H={H}", flush=True)
    g = lrgen.make(5, B=B, L=L, H=H, G=G, N=N, seg=seg)
    h0 = lrgen.state_normal((B, H, 64, N), 5, tensor_id=21, std=0.3)
    dhl = lrgen.state_normal((B, H, 64, N), 5, tensor_id=22, std=0.3)
    T = {k: dev(g.t(k)) for k in ("x", "dt", "A", "B", "C", "Dskip", "dy")}
    h0d, dhld = dev(h0, "f32"), dev(dhl, "f32")
    _, _, ck = lr.lr_ssd_scan(T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"], h0d,
                              disc=disc, seg=seg, want_last=True)
    args = (T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"], h0d, ck, T["dy"], dhld)
    full = lr.lr_ssd_scan_bwd(*args, disc=disc, seg=seg, want_dh0=True)
    small = _one_row_ws(B, L, H, 64, G, N, seg)
    assert small < lr.lr_ssd_scan_bwd_workspace_bytes(B, L, H, 64, G, N, 64, seg)
    ws = torch.empty(small, device="cuda", dtype=torch.uint8)
    part = lr.lr_ssd_scan_bwd(*args, disc=disc, seg=seg, workspace=ws, want_dh0=True)
    torch.cuda.synchronize()
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"):
        assert torch.equal(full[k], part[k]), k
    if disc == "zoh":   # (bilinear parity: test_gpu_disc.py)
        ref = oracle.ssd_scan_bwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], h0,
                                  g["dy"], dhl, disc)
        for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"):
            check(k, full[k], ref[k], TOL["bf16"])
    one_row = lr.lr_ssd_scan_bwd_workspace_bytes(1, L, H, 64, G, N, 64, seg)
    with pytest.raises(lr.LrError, match="LR_E_WORKSPACE"):
        lr.lr_ssd_scan_bwd(*args, disc=disc, seg=seg, want_dh0=True,
                           workspace=torch.empty(one_row // 2, device="cuda", dtype=torch.uint8))
