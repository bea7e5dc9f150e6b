"""GPU parity of the bilinear (Tustin) and dirac discretisations against the
fp64 oracle, through the C ABI: selective scan forward, backward and step,
SSD forward (including decays made negative by the bilinear map), backward
(dirac) and step."""
import numpy as np
import pytest
import torch

import lrgen
import oracle
import ssm_selective_scan_amd as lr
from gpu_util import TOL, check, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("disc", ["bilinear", "dirac"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 28, 50])
def test_selective_fwd_bwd(disc, io, N):
    B, L, D, seg = 2, 300, 70, 64
    print(f"selective {disc} io={io} N={N}", flush=True)
    g = lrgen.make(2, io=io, B=B, L=L, D=D, N=N, grads=True)
    h0 = lrgen.state_normal((B, D, N), 2, tensor_id=21, std=0.5)
    dhl = lrgen.state_normal((B, D, N), 2, tensor_id=22, std=0.5)
    T = {k: dev(g.t(k)) for k in ("x", "dt", "B", "C", "dy")}
    A, Dk = dev(g.t("A")), dev(g.t("Dskip"))
    y, hl, ck = lr.lr_selective_scan(T["x"], T["dt"], A, T["B"], T["C"], Dk, h0=dev(h0, "f32"),
                                     disc=disc, seg=seg, want_last=True)
    gr = lr.lr_selective_scan_bwd(T["x"], T["dt"], A, T["B"], T["C"], Dk, ck, T["dy"],
                                  dev(dhl, "f32"), disc=disc, seg=seg, want_dh0=True)
    torch.cuda.synchronize()
    ry, rh = oracle.selective_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], h0, disc)
    check("y", y, ry, TOL[io])
    check("h_last", hl, rh, TOL[io])
    ref = oracle.selective_scan_bwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], h0,
                                    g["dy"], dhl, disc)
    for name in ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"):
        check(name, gr[name], ref[name], TOL[io])


@pytest.mark.parametrize("disc,dt_scale", [("bilinear", 1.0), ("bilinear", 32.0),
                                           ("dirac", 1.0)])
def test_ssd_fwd(disc, dt_scale):
    """dt_scale = 32 pushes many tokens past dt A = -2, where the bilinear
    decay is negative and the chunked form tracks its sign."""
    B, L, H, P, G, N = 2, 333, 4, 64, 2, 128
    print(f"ssd {disc} dt_scale={dt_scale}", flush=True)
    g = lrgen.make(3, B=B, L=L, H=H, P=P, G=G, N=N)
    dt = lrgen.round_bf16(g["dt"] * dt_scale)   # power-of-two scale keeps bf16 values exact
    h0 = lrgen.state_normal((B, H, P, N), 3, std=0.3)
    y, hl = lr.lr_ssd_scan(dev(g.t("x")), dev(dt, "bf16"), dev(g.t("A")), dev(g.t("B")),
                           dev(g.t("C")), dev(g.t("Dskip")), dev(h0, "f32"), disc=disc,
                           want_last=True)[:2]
    torch.cuda.synchronize()
    ry, rh, _ = oracle.ssd_scan(g["x"], dt, g["A"], g["B"], g["C"], g["Dskip"], h0, disc)
    if disc == "bilinear" and dt_scale > 1:
        e, _ = oracle.discretize(dt, g["A"][None, None], disc)
        assert (e < 0).mean() > 0.05, "the case must contain negative decays"
    check("y", y, ry, TOL["bf16"])
    check("h_last", hl, rh, TOL["bf16"])


def test_ssd_bwd_dirac():
    g = lrgen.make(5, B=2, L=200, H=3, G=1, N=128, seg=128)
    h0 = lrgen.state_normal((2, 3, 64, 128), 5, tensor_id=21, std=0.3)
    T = {k: dev(g.t(k)) for k in ("x", "dt", "A", "B", "C", "Dskip", "dy")}
    y, hl, ck = lr.lr_ssd_scan(T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"],
                               dev(h0, "f32"), disc="dirac", seg=128, want_last=True)
    gr = lr.lr_ssd_scan_bwd(T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"], dev(h0, "f32"),
                            ck, T["dy"], disc="dirac", seg=128, want_dh0=True)
    torch.cuda.synchronize()
    ref = oracle.ssd_scan_bwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], h0, g["dy"],
                              None, "dirac")
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"):
        check(k, gr[k], ref[k], TOL["bf16"])


@pytest.mark.parametrize("dt_scale,seg,dhl", [(1.0, 128, False), (32.0, 64, True),
                                          (32.0, 256, False)])
def test_ssd_bwd_bilinear(dt_scale, seg, dhl):
    """Bilinear SSD backward; dt_scale = 32 gives negative decays, whose signs
    the block algebra tracks as the forward does."""
    B, L, H, G, N = 2, 300, 3, 1, 128
    print(f"ssd bwd bilinear dt_scale={dt_scale} seg={seg} dh_last={dhl}", flush=True)
    g = lrgen.make(5, B=B, L=L, H=H, G=G, N=N, seg=seg)
    dt = lrgen.round_bf16(g["dt"] * dt_scale)   # power-of-two scale keeps bf16 values exact
    h0 = lrgen.state_normal((B, H, 64, N), 5, tensor_id=21, std=0.3)
    dh_last = lrgen.state_normal((B, H, 64, N), 5, tensor_id=22, std=0.3) if dhl else None
    T = {k: dev(g.t(k)) for k in ("x", "A", "B", "C", "Dskip", "dy")}
    dtd = dev(dt, "bf16")
    y, hl, ck = lr.lr_ssd_scan(T["x"], dtd, T["A"], T["B"], T["C"], T["Dskip"], dev(h0, "f32"),
                               disc="bilinear", seg=seg, want_last=True)
    gr = lr.lr_ssd_scan_bwd(T["x"], dtd, T["A"], T["B"], T["C"], T["Dskip"], dev(h0, "f32"), ck,
                            T["dy"], None if dh_last is None else dev(dh_last, "f32"),
                            disc="bilinear", seg=seg, want_dh0=True)
    torch.cuda.synchronize()
    if dt_scale > 1:
        e, _ = oracle.discretize(dt, g["A"][None, None], "bilinear")
        assert (e < 0).mean() > 0.05, "the case must contain negative decays"
    ref = oracle.ssd_scan_bwd(g["x"], dt, g["A"], g["B"], g["C"], g["Dskip"], h0, g["dy"],
                              dh_last, "bilinear")
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0"):
        check(k, gr[k], ref[k], TOL["bf16"])


@pytest.mark.parametrize("disc", ["bilinear", "dirac"])
def test_steps(disc):
    g = lrgen.make(2, io="f32", B=2, L=17, D=64, N=16)
    h = torch.zeros(2, 64, 16, device="cuda")
    X = {k: dev(g.t(k)) for k in ("x", "dt", "B", "C")}
    A, Dk = dev(g.t("A")), dev(g.t("Dskip"))
    ys = [lr.lr_selective_step(X["x"][:, t].contiguous(), X["dt"][:, t].contiguous(), A,
                               X["B"][:, t].contiguous(), X["C"][:, t].contiguous(), Dk, h, disc=disc)
          for t in range(17)]
    gs = lrgen.make(3, B=2, L=17, H=4, P=64, G=1, N=64)
    hs = torch.zeros(2, 4, 64, 64, device="cuda")
    Y = {k: dev(gs.t(k)) for k in ("x", "dt", "B", "C")}
    As, Ds = dev(gs.t("A")), dev(gs.t("Dskip"))
    yss = [lr.lr_ssd_step(Y["x"][:, t].contiguous(), Y["dt"][:, t].contiguous(), As,
                          Y["B"][:, t].contiguous(), Y["C"][:, t].contiguous(), Ds, hs, disc=disc)
           for t in range(17)]
    torch.cuda.synchronize()
    ry, _ = oracle.selective_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], None, disc)
    check("selective step y", torch.stack(ys, 1), ry, TOL["f32"])
    rys, _, _ = oracle.ssd_scan(gs["x"], gs["dt"], gs["A"], gs["B"], gs["C"], gs["Dskip"], None, disc)
    check("ssd step y", torch.stack(yss, 1), rys, TOL["bf16"])
