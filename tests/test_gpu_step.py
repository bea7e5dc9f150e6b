"""GPU parity of the single-token step kernels: T steps from an initial
state reproduce the oracle's scan over the same T tokens (recurrent vs
step-wise mode), match the GPU's own parallel scan, and a captured HIP
graph of a decode loop replays bit-identically to the eager loop."""
import numpy as np
import pytest
import torch

import lrgen
import oracle
import ssm_selective_scan_amd as lr
from gpu_util import TOL, check, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_diag_step(io):
    g = lrgen.make(1, io=io, B=2, L=37, D=300)
    h0 = lrgen.state_normal((2, 300), 1)
    a, b = dev(g.t("a")), dev(g.t("b"))
    h = dev(h0, "f32").clone()
    outs = [lr.lr_diag_step(a[:, t].contiguous(), b[:, t].contiguous(), h) for t in range(37)]
    torch.cuda.synchronize()
    ref, ref_last = oracle.diag_scan(g["a"], g["b"], h0)
    check("h", torch.stack(outs, 1), ref, TOL[io])
    check("state", h, ref_last, TOL["f32"] if io == "f32" else TOL["bf16"])


@pytest.mark.parametrize("io,disc,N", [("f32", "zoh", 16), ("bf16", "zoh", 16),
                                       ("f32", "euler", 5), ("bf16", "zoh", 64)])
def test_selective_step(io, disc, N):
    B, T, D = 2, 29, 130
    g = lrgen.make(2, io=io, B=B, L=T, D=D, N=N, disc=disc)
    h0 = lrgen.state_normal((B, D, N), 2, std=0.5)
    T_ = {k: dev(g.t(k)) for k in ("x", "dt", "B", "C")}
    A, Dk = dev(g.t("A")), dev(g.t("Dskip"))
    h = dev(h0, "f32").clone()
    ys = [lr.lr_selective_step(T_["x"][:, t].contiguous(), T_["dt"][:, t].contiguous(), A,
                               T_["B"][:, t].contiguous(), T_["C"][:, t].contiguous(), Dk, h,
                               disc=disc) for t in range(T)]
    yp, hp = lr.lr_selective_scan(T_["x"], T_["dt"], A, T_["B"], T_["C"], Dk, h0=dev(h0, "f32"),
                                  disc=disc, want_last=True)
    torch.cuda.synchronize()
    ry, rh = oracle.selective_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], h0, disc)
    check("y (steps)", torch.stack(ys, 1), ry, TOL[io])
    check("state (steps)", h, rh, TOL[io])
    check("steps vs parallel scan", host(torch.stack(ys, 1)), host(yp), TOL[io])


@pytest.mark.parametrize("N,G,P", [(128, 1, 64), (64, 2, 64), (128, 1, 5), (64, 1, 3)])
def test_ssd_step(N, G, P):
    B, T, H = 2, 23, 4
    g = lrgen.make(3, B=B, L=T, H=H, P=P, G=G, N=N)
    h0 = lrgen.state_normal((B, H, P, N), 3, std=0.3)
    X = {k: dev(g.t(k)) for k in ("x", "dt", "B", "C")}
    A, Dk = dev(g.t("A")), dev(g.t("Dskip"))
    h = dev(h0, "f32").clone()
    ys = [lr.lr_ssd_step(X["x"][:, t].contiguous(), X["dt"][:, t].contiguous(), A,
                         X["B"][:, t].contiguous(), X["C"][:, t].contiguous(), Dk, h)
          for t in range(T)]
    torch.cuda.synchronize()
    ry, rh, _ = oracle.ssd_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], h0)
    check("y (steps)", torch.stack(ys, 1), ry, TOL["bf16"])
    check("state (steps)", h, rh, TOL["bf16"])


@pytest.mark.parametrize("K,V", [(128, 128), (64, 192), (200, 64), (5, 64)])
def test_gla_step(K, V):
    B, T, H = 2, 21, 3
    g = lrgen.make(4, B=B, L=T, H=H, K=K, V=V)
    S0 = lrgen.state_normal((B, H, K, V), 4, std=0.3)
    X = {k: dev(g.t(k)) for k in ("q", "k", "v", "g")}
    S = dev(S0, "f32").clone()
    os_ = [lr.lr_gla_step(X["q"][:, t].contiguous(), X["k"][:, t].contiguous(),
                          X["v"][:, t].contiguous(), X["g"][:, t].contiguous(), S)
           for t in range(T)]
    torch.cuda.synchronize()
    ro, rS = oracle.gla_scan(g["q"], g["k"], g["v"], g["g"], S0)
    check("o (steps)", torch.stack(os_, 1), ro, TOL["bf16"])
    check("state (steps)", S, rS, TOL["bf16"])


def test_ssd_decode_graph_replays():
    """A 16-step decode loop captured in a graph: each replay (with eager work
    and synchronisation in between) equals the same loop run eagerly."""
    B, T, H, P, G, N = 2, 16, 8, 64, 1, 128
    g = lrgen.make(3, B=B, L=T, H=H, P=P, G=G, N=N)
    xs = [dev(g.t("x"))[:, t].contiguous() for t in range(T)]
    dts = [dev(g.t("dt"))[:, t].contiguous() for t in range(T)]
    Bs = [dev(g.t("B"))[:, t].contiguous() for t in range(T)]
    Cs = [dev(g.t("C"))[:, t].contiguous() for t in range(T)]
    A, Dk = dev(g.t("A")), dev(g.t("Dskip"))
    h = torch.zeros(B, H, P, N, device="cuda")
    ys = [torch.empty(B, H, P, device="cuda", dtype=torch.bfloat16) for _ in range(T)]

    def loop(state, outs):
        for t in range(T):
            lr.lr_ssd_step(xs[t], dts[t], A, Bs[t], Cs[t], Dk, state, y=outs[t])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop(h, ys)                      # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    h.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop(h, ys)
    torch.cuda.synchronize()
    h.zero_()
    h_ref = torch.zeros_like(h)
    ys_ref = [torch.empty_like(y) for y in ys]
    for rep in range(3):
        graph.replay()
        loop(h_ref, ys_ref)              # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(h, h_ref), f"state after replay {rep}"
        for t in range(T):
            assert torch.equal(ys[t], ys_ref[t]), f"y[{t}] after replay {rep}"
