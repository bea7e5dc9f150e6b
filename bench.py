"""Benchmark of the linear-recurrence scans on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the headline workload over one batch of synthetic
input already resident in HBM: the Mamba-1 selective scan with ZOH and fused
readout at B=8, L=4096, D=2048, N=16, bf16 I/O, fp32 state (the workload the
prefill tokens/s metric is quoted on).  W untimed warm-up steps, then K timed
steps bracketed by torch.cuda.synchronize(); the kernel's own duration is
taken with HIP events recorded on the launch stream.  Input/output buffer
sets are rotated so that the 256 MB Infinity Cache cannot hold a step's
working set from the previous step.

Before the warm-ups, the headline kernel runs back to back for --settle-ms
of GPU time (reported as clock_settle), so the timed steps see steady
clocks rather than the first launches' ramp.

The same run also measures the other four workloads (diagonal scan, SSD
forward, GLA forward, SSD forward + backward with segment checkpoints), the
backward and decode paths, and a plain device copy for the achievable
bandwidth; records which kernels each call dispatched (dispatch, from the
torch profiler's HIP activity trace); and, after the GPU work, times the
fp64 CPU oracle on every workload on the host's cores, in worker processes
forked before this process starts the GPU runtime (cpu_baseline: the
headline's figure, with per_workload for all five and the GPU-over-oracle
ratios).  Timing the oracle first slowed the headline's first timed
launches.  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import lrgen  # noqa: E402
import ssm_selective_scan_amd as lr  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
# fp32 VALU issue rate without packed math: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
METRIC = "SSD/selective-scan prefill tokens/s + achieved HBM GB/s vs MI355X peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(t):
    x = torch.from_numpy(np.ascontiguousarray(t.values)).cuda()
    return x.to(torch.bfloat16) if t.io == "bf16" else x


def rotations(nbytes, floor=3):
    """Buffer sets needed so consecutive launches never share a cached set."""
    return max(floor, int(np.ceil(768e6 / max(nbytes, 1))) + 1)


def time_launches(fn, sets, warmup, iters, settle_ms=30.0):
    """Average duration (s) of fn(set) measured with events on the launch
    stream, cycling through the buffer sets, after `settle_ms` of untimed
    back-to-back launches and `warmup` more."""
    stream = torch.cuda.current_stream()
    if settle_ms > 0:
        settle_clocks(fn, sets, settle_ms)
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record(stream)
        fn(sets[i % len(sets)])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return ms.mean() / 1e3, ms


def graph_launch_time(fn, k=50, reps=20):
    """Per-launch time (s) of fn when k launches run back to back from one
    captured HIP graph (replayed `reps` times): the GPU-side cost of a launch
    without host enqueue gaps, which dominate event timings of single
    launches of a few microseconds."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(k):
            fn()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / 1e3 / (k * reps)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
def selective_setup(g):
    x, dt, Bm, Cm = dev(g.t("x")), dev(g.t("dt")), dev(g.t("B")), dev(g.t("C"))
    A, Dk = dev(g.t("A")), dev(g.t("Dskip"))
    per = sum(t.numel() * t.element_size() for t in (x, dt, Bm, Cm)) * 3 // 2
    R = rotations(per)
    sets = [dict(x=x if i == 0 else x.clone(), dt=dt if i == 0 else dt.clone(),
                 Bm=Bm if i == 0 else Bm.clone(), Cm=Cm if i == 0 else Cm.clone(),
                 y=torch.empty_like(x)) for i in range(R)]

    def fn(s):
        lr.lr_selective_scan(s["x"], s["dt"], A, s["Bm"], s["Cm"], Dk, disc="zoh", y=s["y"])
    return fn, sets


def selective_bytes(p):
    B, L, D, N = p["B"], p["L"], p["D"], p["N"]
    return 3 * B * L * D * 2 + 2 * B * L * N * 2 + D * N * 4 + D * 4


def sel_valu_ops(p):
    # fused ZOH update per (b, t, d, n): e = 2^(dt A log2e) (1 mul + 1 exp),
    # v = (B x)/A (2 mul), h = e (h + v) - v (add + fma), y += C h (fma)
    B, L, D, N = p["B"], p["L"], p["D"], p["N"]
    return 7 * B * L * D * N


def measure_diag(warmup, iters):
    g = lrgen.make(1)
    a, b = dev(g.t("a")), dev(g.t("b"))
    sets = [dict(a=a, b=b, h=torch.empty_like(a))]
    call = lambda s: lr.lr_diag_scan(s["a"], s["b"], h=s["h"])
    te, _ = time_launches(call, sets, warmup, iters)
    t = graph_launch_time(lambda: call(sets[0]))
    p = g.params
    nb = 3 * p["B"] * p["L"] * p["D"] * 4
    return dict(workload=lrgen.NAMES[1], kernels=fingerprint(lambda: call(sets[0])), us=t * 1e6,
                us_event_single_launch=te * 1e6, trivial_kernel_us=trivial_kernel_times(),
                tokens_per_s=p["B"] * p["L"] / t, elems_per_s=p["B"] * p["L"] * p["D"] / t,
                alg_bytes=nb, GBs=nb / t / 1e9, hbm_frac=nb / t / 1e9 / HBM_PEAK_GBS,
                note="3 MB working set: launch/latency bound; us is the per-launch time of 50 "
                     "launches back to back in one graph, us_event_single_launch brackets one "
                     "launch with events (includes host enqueue gaps)")


def trivial_kernel_times():
    """The same two timings of a one-element torch kernel: the floor of each
    method on this machine."""
    z = torch.zeros(1, device="cuda")
    te, _ = time_launches(lambda s: z.add_(1.0), [None], 50, 200, settle_ms=0)
    return dict(us=graph_launch_time(lambda: z.add_(1.0)) * 1e6, us_event_single_launch=te * 1e6)


def measure_ssd(warmup, iters):
    g = lrgen.make(3)
    p = g.params
    x, dt, Bm, Cm = dev(g.t("x")), dev(g.t("dt")), dev(g.t("B")), dev(g.t("C"))
    A, Dk = dev(g.t("A")), dev(g.t("Dskip"))
    per = sum(t.numel() * t.element_size() for t in (x, dt, Bm, Cm)) + x.numel() * 2
    sets = [dict(x=x if i == 0 else x.clone(), dt=dt if i == 0 else dt.clone(),
                 Bm=Bm if i == 0 else Bm.clone(), Cm=Cm if i == 0 else Cm.clone(),
                 y=torch.empty_like(x)) for i in range(rotations(per))]
    B, L, H, P, N = p["B"], p["L"], p["H"], p["P"], p["N"]
    wsb = lr.lr_ssd_scan_workspace_bytes(B, L, H, P, p["G"], N, p["chunk"])
    ws = torch.empty(wsb, device="cuda", dtype=torch.uint8) if wsb else None
    call = lambda s: lr.lr_ssd_scan(s["x"], s["dt"], A, s["Bm"], s["Cm"], Dk, chunk=p["chunk"],
                                    y=s["y"], workspace=ws)
    t, _ = time_launches(call, sets, warmup, iters)
    nb = 2 * B * L * H * P * 2 + B * L * H * 2 + 2 * B * L * N * 2 + 2 * H * 4
    fl = ssd_mfma_flops(B, L, H, P, N)
    return dict(workload=lrgen.NAMES[3], kernels=fingerprint(lambda: call(sets[0])),
                fwd_workspace_bytes=wsb, us=t * 1e6,
                tokens_per_s=B * L / t, elems_per_s=B * L * H * P / t, alg_bytes=nb,
                GBs=nb / t / 1e9, hbm_frac=nb / t / 1e9 / HBM_PEAK_GBS,
                mfma_tflops=fl / t / 1e12, mfma_frac=fl / t / 1e12 / MFMA_BF16_PEAK_TFLOPS)


def ssd_mfma_flops(B, L, H, P, N, Q=64):
    # MFMA work of the 64-token block form per (b, h, block): C B^T on the
    # causal 10 of 16 tiles, M X (causal), C h_prev, B_w^T X
    per_blk = 2 * (10 * 16 * 16 * N + (Q * Q // 2 + Q * 8) * P + Q * N * P + N * Q * P)
    return B * H * ((L + Q - 1) // Q) * per_blk


def measure_gla(warmup, iters):
    g = lrgen.make(4)
    p = g.params
    q, k, v, gg = dev(g.t("q")), dev(g.t("k")), dev(g.t("v")), dev(g.t("g"))
    per = 4 * q.numel() * 2
    sets = [dict(q=q if i == 0 else q.clone(), k=k if i == 0 else k.clone(),
                 v=v if i == 0 else v.clone(), g=gg, o=torch.empty_like(v))
            for i in range(rotations(per, floor=2))]
    B, L, H, K, V = p["B"], p["L"], p["H"], p["K"], p["V"]
    wsb = lr.lr_gla_scan_workspace_bytes(B, L, H, K, V, p["chunk"])
    ws = torch.empty(wsb, device="cuda", dtype=torch.uint8) if wsb else None
    call = lambda s: lr.lr_gla_scan(s["q"], s["k"], s["v"], s["g"], chunk=p["chunk"], o=s["o"],
                                    workspace=ws)
    t, _ = time_launches(call, sets, warmup, iters)
    nb = 2 * B * L * H * K * 2 + 2 * B * L * H * V * 2 + B * L * H * 2
    fl = (V // 64) * ssd_mfma_flops(B, L, H, 64, K)
    return dict(workload=lrgen.NAMES[4], kernels=fingerprint(lambda: call(sets[0])),
                fwd_workspace_bytes=wsb, us=t * 1e6,
                tokens_per_s=B * L / t, elems_per_s=B * L * H * V / t, alg_bytes=nb,
                GBs=nb / t / 1e9, hbm_frac=nb / t / 1e9 / HBM_PEAK_GBS,
                mfma_tflops=fl / t / 1e12, mfma_frac=fl / t / 1e12 / MFMA_BF16_PEAK_TFLOPS)


def measure_ssd_bwd(warmup, iters):
    g = lrgen.make(5)
    p = g.params
    B, L, H, P, G, N, seg = p["B"], p["L"], p["H"], p["P"], p["G"], p["N"], p["seg"]
    x, dt, Bm, Cm = dev(g.t("x")), dev(g.t("dt")), dev(g.t("B")), dev(g.t("C"))
    A, Dk, dy = dev(g.t("A")), dev(g.t("Dskip")), dev(g.t("dy"))
    y = torch.empty_like(x)
    nseg = (L + seg - 1) // seg
    ckpt = torch.empty(nseg, B, H, P, N, device="cuda", dtype=torch.float32)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    fwsb = lr.lr_ssd_scan_workspace_bytes(B, L, H, P, G, N, p["chunk"])
    fws = torch.empty(fwsb, device="cuda", dtype=torch.uint8) if fwsb else None
    fcall = lambda s: lr.lr_ssd_scan(x, dt, A, Bm, Cm, Dk, chunk=p["chunk"], seg=seg, y=y,
                                     ckpt=ckpt, workspace=fws)
    tf, _ = time_launches(fcall, [None], warmup, iters)
    ws_bytes = lr.lr_ssd_scan_bwd_workspace_bytes(B, L, H, P, G, N, p["chunk"], seg)
    # state-related memory: checkpoints, the forward's part states, the backward's workspace
    out = dict(workload=lrgen.NAMES[5], fwd_us=tf * 1e6,
               ckpt_bytes=ckpt.numel() * 4,
               full_state_bytes=L * B * H * P * N * 4,
               state_mem_ratio=(L * B * H * P * N * 4) / (ckpt.numel() * 4 + ws_bytes + fwsb),
               fwd_workspace_bytes=fwsb, bwd_workspace_bytes=ws_bytes)
    fwd_bytes = 2 * B * L * H * P * 2 + B * L * H * 2 + 2 * B * L * N * 2 + ckpt.numel() * 4
    out["fwd_GBs"] = fwd_bytes / tf / 1e9
    try:
        ws = torch.empty(max(ws_bytes, 16), device="cuda", dtype=torch.uint8)
        bcall = lambda s: lr.lr_ssd_scan_bwd(x, dt, A, Bm, Cm, Dk, None, ckpt, dy,
                                             chunk=p["chunk"], seg=seg, workspace=ws)
        tb, _ = time_launches(bcall, [None], warmup, iters)
        bwd_bytes = (3 * B * L * H * P * 2 + 2 * B * L * H * 2 + 4 * B * L * N * 2
                     + ckpt.numel() * 4)
        out.update(kernels=fingerprint(lambda: (fcall(None), bcall(None))),
                   bwd_us=tb * 1e6, bwd_GBs=bwd_bytes / tb / 1e9,
                   fwd_bwd_tokens_per_s=B * L / (tf + tb),
                   peak_alloc_delta_bytes=torch.cuda.max_memory_allocated() - base)
    except lr.LrError as e:
        out["bwd"] = f"unavailable: {e}"
    return out


def measure_rotlru(warmup, iters):
    g = lrgen.make(6)
    r, th, u = dev(g.t("r")), dev(g.t("theta")), dev(g.t("u"))
    h = torch.empty_like(u)
    fcall = lambda: lr.lr_rotlru_scan(r, th, u, h=h)
    te, _ = time_launches(lambda s: fcall(), [None], warmup, iters)
    t = graph_launch_time(fcall)
    p = g.params
    nb = 2 * p["B"] * p["L"] * p["D"] * 4 + 2 * p["B"] * p["L"] * (p["D"] // 2) * 4
    out = dict(workload=lrgen.NAMES[6], kernels=fingerprint(fcall), us=t * 1e6,
               us_event_single_launch=te * 1e6,
               tokens_per_s=p["B"] * p["L"] / t, elems_per_s=p["B"] * p["L"] * p["D"] / t,
               alg_bytes=nb, GBs=nb / t / 1e9, hbm_frac=nb / t / 1e9 / HBM_PEAK_GBS,
               note="3 MB working set: launch/latency bound")
    dh = dev(lrgen.make(6, grads=True).t("dh"))
    bcall = lambda: lr.lr_rotlru_scan_bwd(r, th, h, dh)
    tbe, _ = time_launches(lambda s: bcall(), [None], warmup, iters)
    tb = graph_launch_time(bcall)
    # read r, theta, h, dh; write dr, dtheta, du
    nbb = 3 * p["B"] * p["L"] * p["D"] * 4 + 4 * p["B"] * p["L"] * (p["D"] // 2) * 4
    out.update(bwd_kernels=fingerprint(bcall), bwd_us=tb * 1e6,
               bwd_us_event_single_launch=tbe * 1e6, bwd_alg_bytes=nbb, bwd_GBs=nbb / tb / 1e9)
    return out



def measure_scaled(warmup, iters):
    """Labelled scaled sweep of the two elementwise scans (diagonal and
    rotational LRU), whose small workloads are launch bound: B=16, L=8192,
    D=4096, fp32, seeded uniform/normal inputs of the small workloads'
    distributions.  Reports the algorithmic HBM bandwidth of each kernel."""
    B, L, D = 16, 8192, 4096
    gen = torch.Generator(device="cuda").manual_seed(2026)
    a = torch.empty(B, L, D, device="cuda").uniform_(0.90, 0.999, generator=gen)
    b = torch.randn(B, L, D, device="cuda", generator=gen)
    h = torch.empty_like(a)
    t, _ = time_launches(lambda s: lr.lr_diag_scan(a, b, h=h), [None], warmup, iters)
    nb = 3 * B * L * D * 4
    out = {"diag": dict(shape=f"B{B}_L{L}_D{D}_fp32", us=t * 1e6, alg_bytes=nb, GBs=nb / t / 1e9,
                        hbm_frac=nb / t / 1e9 / HBM_PEAK_GBS)}
    t, _ = time_launches(lambda s: lr.lr_diag_scan_bwd(a, h, b), [None], warmup, iters)
    nb = 5 * B * L * D * 4     # read a, h, dh; write da, db
    out["diag_bwd"] = dict(shape=f"B{B}_L{L}_D{D}_fp32", us=t * 1e6, alg_bytes=nb,
                           GBs=nb / t / 1e9, hbm_frac=nb / t / 1e9 / HBM_PEAK_GBS)
    th = torch.empty(B, L, D // 2, device="cuda").uniform_(-np.pi, np.pi, generator=gen)
    r = a[:, :, :D // 2].contiguous()
    t, _ = time_launches(lambda s: lr.lr_rotlru_scan(r, th, b, h=h), [None], warmup, iters)
    nb = 2 * B * L * D * 4 + 2 * B * L * (D // 2) * 4
    out["rotlru"] = dict(shape=f"B{B}_L{L}_D{D}_fp32", us=t * 1e6, alg_bytes=nb,
                         GBs=nb / t / 1e9, hbm_frac=nb / t / 1e9 / HBM_PEAK_GBS)
    t, _ = time_launches(lambda s: lr.lr_rotlru_scan_bwd(r, th, h, b), [None], warmup, iters)
    nb = 3 * B * L * D * 4 + 4 * B * L * (D // 2) * 4   # read r, theta, h, dh; write dr, dtheta, du
    out["rotlru_bwd"] = dict(shape=f"B{B}_L{L}_D{D}_fp32", us=t * 1e6, alg_bytes=nb,
                             GBs=nb / t / 1e9, hbm_frac=nb / t / 1e9 / HBM_PEAK_GBS)
    return out

def measure_diag_bwd(warmup, iters):
    g = lrgen.make(1, grads=True)
    a, b, dh = dev(g.t("a")), dev(g.t("b")), dev(g.t("dh"))
    h, _ = lr.lr_diag_scan(a, b)
    call = lambda: lr.lr_diag_scan_bwd(a, h, dh)
    te, _ = time_launches(lambda s: call(), [None], warmup, iters)
    t = graph_launch_time(call)
    p = g.params
    nb = 5 * p["B"] * p["L"] * p["D"] * 4     # read a, h, dh; write da, db
    return dict(workload=lrgen.NAMES[1] + "_bwd", kernels=fingerprint(call), us=t * 1e6,
                us_event_single_launch=te * 1e6,
                tokens_per_s=p["B"] * p["L"] / t, alg_bytes=nb, GBs=nb / t / 1e9,
                hbm_frac=nb / t / 1e9 / HBM_PEAK_GBS,
                note="5 MB working set: launch/latency bound; timings as for diag")


def measure_selective_bwd(warmup, iters):
    """Mamba-1 workload, forward with segment checkpoints (seg 256) then the
    backward from them."""
    g = lrgen.make(2, grads=True)
    p = g.params
    B, L, D, N, seg = p["B"], p["L"], p["D"], p["N"], 256
    x, dt, Bm, Cm = dev(g.t("x")), dev(g.t("dt")), dev(g.t("B")), dev(g.t("C"))
    A, Dk, dy = dev(g.t("A")), dev(g.t("Dskip")), dev(g.t("dy"))
    y = torch.empty_like(x)
    ckpt = torch.empty((L + seg - 1) // seg, B, D, N, device="cuda", dtype=torch.float32)
    tf, _ = time_launches(lambda s: lr.lr_selective_scan(x, dt, A, Bm, Cm, Dk, seg=seg, y=y,
                                                         ckpt=ckpt), [None], warmup, iters)
    ws = torch.empty(max(lr.lr_selective_scan_bwd_workspace_bytes(B, L, D, N, seg), 16),
                     device="cuda", dtype=torch.uint8)
    tb, _ = time_launches(lambda s: lr.lr_selective_scan_bwd(x, dt, A, Bm, Cm, Dk, ckpt, dy,
                                                             seg=seg, workspace=ws),
                          [None], warmup, iters)
    bwd_bytes = 5 * B * L * D * 2 + 4 * B * L * N * 2 + ckpt.numel() * 4
    out = dict(workload=lrgen.NAMES[2] + "_fwd_bwd_seg256", fwd_us=tf * 1e6, bwd_us=tb * 1e6,
               fwd_bwd_tokens_per_s=B * L / (tf + tb), bwd_GBs=bwd_bytes / tb / 1e9,
               ckpt_bytes=ckpt.numel() * 4, full_state_bytes=L * B * D * N * 4,
               bwd_workspace_bytes=ws.numel())
    # the other end of the memory/compute trade: a checkpoint every 32 tokens
    # (8x the checkpoint memory) spares the backward its segment forward pass
    del ckpt, ws
    s32 = 32
    ck32 = torch.empty((L + s32 - 1) // s32, B, D, N, device="cuda", dtype=torch.float32)
    tf32, _ = time_launches(lambda s: lr.lr_selective_scan(x, dt, A, Bm, Cm, Dk, seg=s32, y=y,
                                                           ckpt=ck32), [None], warmup, iters)
    ws32 = torch.empty(max(lr.lr_selective_scan_bwd_workspace_bytes(B, L, D, N, s32), 16),
                       device="cuda", dtype=torch.uint8)
    tb32, _ = time_launches(lambda s: lr.lr_selective_scan_bwd(x, dt, A, Bm, Cm, Dk, ck32, dy,
                                                               seg=s32, workspace=ws32),
                            [None], warmup, iters)
    out["seg32"] = dict(fwd_us=tf32 * 1e6, bwd_us=tb32 * 1e6,
                        fwd_bwd_tokens_per_s=B * L / (tf32 + tb32), ckpt_bytes=ck32.numel() * 4,
                        bwd_workspace_bytes=ws32.numel())
    return out


def measure_gla_bwd(warmup, iters):
    """GLA workload, forward with segment checkpoints (seg 256) then the
    backward from them."""
    g = lrgen.make(4, grads=True)
    p = g.params
    B, L, H, K, V, seg = p["B"], p["L"], p["H"], p["K"], p["V"], 256
    q, k, v, gg, do = (dev(g.t(n)) for n in ("q", "k", "v", "g", "do"))
    o = torch.empty_like(v)
    ckpt = torch.empty((L + seg - 1) // seg, B, H, V, K, device="cuda", dtype=torch.float32)
    fwsb = lr.lr_gla_scan_workspace_bytes(B, L, H, K, V, p["chunk"])
    fws = torch.empty(fwsb, device="cuda", dtype=torch.uint8) if fwsb else None
    tf, _ = time_launches(lambda s: lr.lr_gla_scan(q, k, v, gg, chunk=p["chunk"], seg=seg, o=o,
                                                   ckpt=ckpt, workspace=fws), [None], warmup, iters)
    ws = torch.empty(max(lr.lr_gla_scan_bwd_workspace_bytes(B, L, H, K, V, p["chunk"], seg), 16),
                     device="cuda", dtype=torch.uint8)
    tb, _ = time_launches(lambda s: lr.lr_gla_scan_bwd(q, k, v, gg, ckpt, do, chunk=p["chunk"],
                                                       seg=seg, workspace=ws),
                          [None], warmup, iters)
    bwd_bytes = 4 * B * L * H * K * 2 + 3 * B * L * H * V * 2 + 2 * B * L * H * 2 + ckpt.numel() * 4
    return dict(workload=lrgen.NAMES[4] + "_fwd_bwd_seg256", fwd_us=tf * 1e6, bwd_us=tb * 1e6,
                fwd_bwd_tokens_per_s=B * L / (tf + tb), bwd_GBs=bwd_bytes / tb / 1e9,
                ckpt_bytes=ckpt.numel() * 4, full_state_bytes=L * B * H * K * V * 4,
                bwd_workspace_bytes=ws.numel())


def measure_decode(warmup, iters, T=64):
    """Decode: T single-token steps captured in one HIP graph, for the SSD,
    GLA and Mamba-1 state shapes of the prefill workloads.  Reports the time
    per step (graph replay / T), batch tokens/s and the state bytes moved
    (read + write of the fp32 state) per second."""
    out = {}
    gs = lrgen.make(3, L=T)
    ps = gs.params
    B, H, P, N = ps["B"], ps["H"], ps["P"], ps["N"]
    X = {k: dev(gs.t(k)) for k in ("x", "dt", "B", "C")}
    A, Dk = dev(gs.t("A")), dev(gs.t("Dskip"))
    steps_ssd = [tuple(X[k][:, t].contiguous() for k in ("x", "dt", "B", "C")) for t in range(T)]
    h = torch.zeros(B, H, P, N, device="cuda")
    ys = [torch.empty(B, H, P, device="cuda", dtype=torch.bfloat16) for _ in range(T)]
    ssd_loop = lambda: [lr.lr_ssd_step(x, d, A, b, c, Dk, h, y=ys[t])
                        for t, (x, d, b, c) in enumerate(steps_ssd)]

    gg = lrgen.make(4, L=T)
    pg = gg.params
    Bg, Hg, K, V = pg["B"], pg["H"], pg["K"], pg["V"]
    Y = {k: dev(gg.t(k)) for k in ("q", "k", "v", "g")}
    steps_gla = [tuple(Y[k][:, t].contiguous() for k in ("q", "k", "v", "g")) for t in range(T)]
    S = torch.zeros(Bg, Hg, K, V, device="cuda")
    os_ = [torch.empty(Bg, Hg, V, device="cuda", dtype=torch.bfloat16) for _ in range(T)]
    gla_loop = lambda: [lr.lr_gla_step(q, k, v, g_, S, o=os_[t])
                        for t, (q, k, v, g_) in enumerate(steps_gla)]

    gm = lrgen.make(2, L=T)
    pm = gm.params
    Bm_, D, Nm = pm["B"], pm["D"], pm["N"]
    Z = {k: dev(gm.t(k)) for k in ("x", "dt", "B", "C")}
    Am, Dm = dev(gm.t("A")), dev(gm.t("Dskip"))
    steps_sel = [tuple(Z[k][:, t].contiguous() for k in ("x", "dt", "B", "C")) for t in range(T)]
    hm = torch.zeros(Bm_, D, Nm, device="cuda")
    yms = [torch.empty(Bm_, D, device="cuda", dtype=torch.bfloat16) for _ in range(T)]
    sel_loop = lambda: [lr.lr_selective_step(x, d, Am, b, c, Dm, hm, y=yms[t])
                        for t, (x, d, b, c) in enumerate(steps_sel)]

    for name, loop, batch, state_bytes in (
            ("ssd", ssd_loop, B, h.numel() * 4), ("gla", gla_loop, Bg, S.numel() * 4),
            ("selective", sel_loop, Bm_, hm.numel() * 4)):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            loop()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            loop()
        t, _ = time_launches(lambda s: graph.replay(), [None], warmup, iters)
        ts = t / T
        out[name] = dict(steps_per_graph=T, us_per_step=ts * 1e6, tokens_per_s=batch / ts,
                         state_bytes=state_bytes, state_GBs=2 * state_bytes / ts / 1e9,
                         state_hbm_frac=2 * state_bytes / ts / 1e9 / HBM_PEAK_GBS)
        del graph
    return out


def copy_bandwidth(nbytes=1 << 30, iters=10):
    a = torch.empty(nbytes // 4, device="cuda", dtype=torch.float32).fill_(1.0)
    b = torch.empty_like(a)
    t, _ = time_launches(lambda s: b.copy_(a), [None], 3, iters)
    return 2 * nbytes / t / 1e9


# --------------------------------------------------------------------------
# CPU oracle baselines: every workload, on the host's cores
# --------------------------------------------------------------------------
# Each worker process generates one sample unit of a workload (the recipe of
# lrgen at the unit's shape: a batch row of channels, or one (batch, head)),
# waits at a barrier, runs the fp64 oracle on it with one BLAS thread and
# reports its start and end.  The wall time of the parallel section, scaled
# by (units in the workload) / (units run), is the oracle's time for the
# whole workload on those cores.
#   workload id: (unit shape overrides, units in the workload, what is timed)
CPU_UNITS = {
    1: (dict(), 1, "diag scan, the whole workload"),
    2: (dict(B=1, D=512), 8 * 2048 // 512, "selective scan, one batch row x 512 channels"),
    3: (dict(B=1, H=8), 8 * 32 // 8, "SSD scan, one batch row x 8 heads"),
    4: (dict(B=1, H=4), 8 * 16 // 4, "GLA scan, one batch row x 4 heads"),
    5: (dict(B=1, H=1), 4 * 32, "SSD forward with checkpoints + backward, one (batch, head)"),
}


def _oracle_unit(cfg_id):
    import oracle  # the oracle is test infrastructure; only this leg uses it
    over = CPU_UNITS[cfg_id][0]
    g = lrgen.make(cfg_id, **over)
    if cfg_id == 1:
        return lambda: oracle.diag_scan(g["a"], g["b"])
    if cfg_id == 2:
        return lambda: oracle.selective_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"])
    if cfg_id == 3:
        return lambda: oracle.ssd_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"])
    if cfg_id == 4:
        return lambda: oracle.gla_scan(g["q"], g["k"], g["v"], g["g"])

    def fwd_bwd():
        oracle.ssd_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], seg=g.params["seg"])
        oracle.ssd_scan_bwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["Dskip"], None, g["dy"])
    return fwd_bwd


def _cpu_worker(args):
    cfg_id, reps = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        run = _oracle_unit(cfg_id)
        t0 = time.perf_counter()   # CLOCK_MONOTONIC: comparable across processes
        for _ in range(reps):
            run()
        return t0, time.perf_counter()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_pool(workers):
    """The oracle's worker processes, forked now (before the GPU runtime
    starts in this process) and used at the end by cpu_baselines."""
    import multiprocessing as mp
    return mp.get_context("fork").Pool(workers)


def cpu_baselines(pool, workers):
    """Oracle tokens/s of every workload on `workers` processes, each running
    units // workers units of the workload one after another (all of it when
    the units divide evenly; the diagonal workload, a few milliseconds, on one
    process).  Wall time: first start to last end over the processes."""
    out = {}
    for cfg_id, (_, units, what) in CPU_UNITS.items():
        P = 1 if units == 1 else min(workers, units)
        reps = max(1, units // P)
        spans = pool.map(_cpu_worker, [(cfg_id, reps)] * P, chunksize=1)
        wall = max(e for _, e in spans) - min(s for s, _ in spans)
        p = lrgen.CONFIGS[cfg_id]
        done = P * reps
        full_s = wall * units / done
        tokens = p["B"] * p["L"]
        scaled = "" if done == units else f"; time scaled by {units}/{done}"
        out[lrgen.NAMES[cfg_id]] = dict(
            value=tokens / full_s, unit="tokens/s", cores=P, kind="oracle",
            oracle_s_full_workload=full_s, wall_s=wall,
            sample=f"{done} of {units} units ({what}), full L={p['L']}, fp64 numpy, "
                   f"{P} process{'es' if P > 1 else ''} with one BLAS thread each{scaled}")
        log(f"[bench] oracle {lrgen.NAMES[cfg_id]}: {done} units in {wall:.2f} s on {P} cores "
            f"-> {tokens / full_s:.4g} tokens/s for the whole workload")
    return out


def load_traffic():
    """HBM traffic of the selective kernel from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "selective_scan_mamba1_B8_L4096_D2048_N16_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = read_kv(path)
    if kv.get("kernel_src_sha256_16") != src_hash(("selective_scan.hip", "common.hpp")):
        return None
    return float(kv["traffic_bytes_per_launch"])


SECONDARY_WARMUP, SECONDARY_ITERS = 10, 20


def fingerprint(fn):
    return dispatch_fingerprint({"call": fn})["call"]


# rocprofv3 counter summaries per workload: profiles/<file> holds key = value
# lines; they are attached to the workload only while their source hash
# matches the current sources of the kernels involved
COUNTER_PROFILES = {
    "ssd": ("ssd_fwd_B8_H32_P64_N128_L2048_counters.txt", ("chunk_scan.hip", "common.hpp")),
    "gla": ("gla_fwd_B8_H16_K128_V128_L4096_counters.txt", ("chunk_scan.hip", "common.hpp")),
    "ssd_fwd_bwd": ("ssd_fwd_bwd_B4_H32_P64_N128_L8192_seg256_counters.txt",
                    ("chunk_scan.hip", "ssd_bwd.hip", "common.hpp")),
    "diag": ("diag_B1_L1024_D256_counters.txt", ("diag_scan.hip", "common.hpp")),
}


def src_hash(files):
    import hashlib
    csrc = os.path.join(ROOT, "ssm_selective_scan_amd", "csrc")
    data = b"".join(open(os.path.join(csrc, f), "rb").read() for f in files)
    return hashlib.sha256(data).hexdigest()[:16]


def read_kv(path):
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    return kv


def attach_profiles(extra):
    for key, (fname, files) in COUNTER_PROFILES.items():
        path = os.path.join(ROOT, "profiles", fname)
        if key not in extra or not os.path.exists(path):
            continue
        kv = read_kv(path)
        if kv.get("kernel_src_sha256_16") != src_hash(files):
            extra[key]["counters"] = f"profiles/{fname}: stale (kernel sources changed since)"
            continue
        vals = {}
        for k, v in kv.items():
            if k == "kernel_src_sha256_16":
                continue
            try:
                vals[k] = float(v)
            except ValueError:
                vals[k] = v
        extra[key]["counters"] = dict(vals, source=f"profiles/{fname}")


SECONDARY = {"diag": measure_diag, "ssd": measure_ssd, "gla": measure_gla,
             "ssd_fwd_bwd": measure_ssd_bwd, "diag_bwd": measure_diag_bwd,
             "selective_fwd_bwd": measure_selective_bwd, "gla_fwd_bwd": measure_gla_bwd,
             "decode": measure_decode, "rotlru": measure_rotlru, "scaled": measure_scaled}


def settle_clocks(fn, sets, ms):
    """Run fn back to back for about `ms` milliseconds of GPU time (untimed)
    so the clocks have left their idle state before the warm-up steps."""
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn(sets[i % len(sets)])
            i += 1
        torch.cuda.synchronize()
    return i


def dispatch_fingerprint(calls):
    """Names of the GPU kernels each call dispatches, recorded in-process by
    the torch profiler (HIP activity tracing): the kernels that ran, not the
    ones the code meant to run."""
    from torch.profiler import ProfilerActivity, profile
    out = {}
    for name, fn in calls.items():
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            fn()
            torch.cuda.synchronize()
        names = []
        for ev in prof.events():
            if ev.device_type != torch.autograd.DeviceType.CUDA:
                continue
            nm = ev.name.split("(")[0].replace("void ", "")   # template, no argument list
            if nm not in names:
                names.append(nm)
        out[name] = names
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    # the first few dozen launches of a process run 5-10 % slow while the
    # clocks ramp up; this much back-to-back GPU work precedes the warm-ups
    ap.add_argument("--settle-ms", type=float, default=300.0)
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload (for profiler runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (0: the cores this process may run on, "
                         "at most 16, the host share of one GPU)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--only", choices=sorted(SECONDARY),
                    help="only time one secondary workload (for profiler runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the scans shard by batch/head with no exchange, see DESIGN.md", file=sys.stderr)
        sys.exit(2)

    # the oracle's worker processes are forked before this process starts the
    # GPU runtime; they run the oracle after the GPU measurements
    pool, workers = None, 0
    if not (args.no_cpu or args.copy_probe or args.only or args.headline_only):
        workers = args.cpu_workers or min(len(os.sched_getaffinity(0)), 16)
        pool = cpu_pool(workers)

    if not torch.cuda.is_available():
        print("bench.py: no GPU available", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_probe:
        bw = copy_bandwidth()
        print(json.dumps({"copy_probe_GBs": bw, "bytes_per_copy": 2 * (1 << 30)}))
        return
    if args.only:
        print(json.dumps({args.only: SECONDARY[args.only](args.warmup, args.steps)}))
        return

    log(f"[bench] liblr: {lr.lr_version()}")
    g = lrgen.make(2)
    p = g.params
    fn, sets = selective_setup(g)
    log(f"[bench] headline {lrgen.NAMES[2]}: {len(sets)} rotating buffer sets")

    settle = settle_clocks(fn, sets, args.settle_ms)
    for i in range(args.warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        fn(sets[i % len(sets)])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_step = wall * 1e3 / args.steps
    tokens = p["B"] * p["L"]
    log(f"[bench] headline: {ms_step:.3f} ms/step wall, kernel {kern_ms.mean() * 1e3:.1f} us "
        f"(min {kern_ms.min() * 1e3:.1f}, max {kern_ms.max() * 1e3:.1f})")

    # repeated-experiment protocol of the lrnnx benchmarks: 10 warm-ups, then
    # 90 timed launches, 5 experiments; mean and std of the experiment means
    exp_means, all_ms = [], []
    for _ in range(5):
        _, ms = time_launches(fn, sets, 10, 90)
        exp_means.append(ms.mean())
        all_ms.append(ms)
    all_ms = np.concatenate(all_ms)
    protocol = {"experiments": 5, "warmup": 10, "launches": 90,
                "mean_us": float(np.mean(exp_means) * 1e3),
                "std_us": float(np.std(exp_means) * 1e3),
                "median_us": float(np.median(all_ms) * 1e3)}
    log(f"[bench] protocol: {protocol}")

    fp = {}
    if not args.headline_only:
        fp = dispatch_fingerprint({"headline": lambda: fn(sets[0])})
        log(f"[bench] headline dispatches: {fp['headline']}")

    kt = kern_ms.mean() / 1e3
    nbytes = selective_bytes(p)
    ops = sel_valu_ops(p)
    traffic = load_traffic()
    roofline = {"bound": "alu", "achieved": ops / kt / 1e12, "peak": VALU_PEAK_TOPS,
                "unit": "Tops/s (fp32 VALU lane-ops)",
                "frac": ops / kt / 1e12 / VALU_PEAK_TOPS, "traffic": traffic,
                "kernel": fp["headline"][0] if fp.get("headline") else
                          "lr::selective_pair_kernel (not fingerprinted in this run)",
                "alg_ops_per_launch": ops, "alg_bytes_per_launch": nbytes,
                "hbm_GBs": nbytes / kt / 1e9, "hbm_frac": nbytes / kt / 1e9 / HBM_PEAK_GBS}

    result = {
        "metric": METRIC, "value": tokens / (ms_step / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": lrgen.NAMES[2], "B": p["B"], "L": p["L"], "D": p["D"],
                   "N": p["N"], "io": "bf16", "state": "f32", "disc": "zoh"},
        "kernel_us": kern_ms.mean() * 1e3,
        "kernel_protocol": protocol,
        "clock_settle": {"ms": args.settle_ms, "launches": settle},
        "roofline": roofline,
    }
    del sets
    torch.cuda.empty_cache()

    if not args.headline_only:
        extra = {}
        for name, f in SECONDARY.items():
            log(f"[bench] measuring {name}")
            try:
                extra[name] = f(SECONDARY_WARMUP, SECONDARY_ITERS)
            except Exception as e:  # report, keep the headline line
                extra[name] = {"error": repr(e)}
            torch.cuda.empty_cache()
        extra["copy_GBs"] = copy_bandwidth()
        attach_profiles(extra)
        result["workloads"] = extra
        result["dispatch"] = dict(fp, **{k: v["kernels"] for k, v in extra.items()
                                         if isinstance(v, dict) and "kernels" in v})

    cpu = None
    if pool is not None:
        log(f"[bench] CPU oracle baselines on {workers} worker processes ({cpu_model()})")
        cpu = cpu_baselines(pool, workers)
        pool.close()
        pool.join()
    if cpu is not None:
        head = cpu[lrgen.NAMES[2]]
        result["cpu_baseline"] = dict(head, cpu_model=cpu_model(), per_workload=cpu)
        gpu_tps = {lrgen.NAMES[2]: result["value"]}
        wl = result.get("workloads", {})
        for key, name in (("diag", 1), ("ssd", 3), ("gla", 4)):
            if "tokens_per_s" in wl.get(key, {}):
                gpu_tps[lrgen.NAMES[name]] = wl[key]["tokens_per_s"]
        if "fwd_bwd_tokens_per_s" in wl.get("ssd_fwd_bwd", {}):
            gpu_tps[lrgen.NAMES[5]] = wl["ssd_fwd_bwd"]["fwd_bwd_tokens_per_s"]
        for name, v in cpu.items():
            if name in gpu_tps:
                v["gpu_over_oracle"] = gpu_tps[name] / v["value"]
    print(json.dumps(result))


if __name__ == "__main__":
    main()
