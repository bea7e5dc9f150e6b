"""Dispatch fingerprints: the kernels each workload's call actually runs,
recorded in-process by the torch profiler's HIP activity trace, must be the
ones the design names (a silent switch to another kernel instance, or an
extra launch, fails here)."""
import pytest
import torch
from torch.profiler import ProfilerActivity, profile

import lrgen
import ssm_selective_scan_amd as lr
from gpu_util import dev

pytestmark = pytest.mark.gpu


def kernels(fn):
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    out = []
    for ev in prof.events():
        if ev.device_type == torch.autograd.DeviceType.CUDA:
            out.append(ev.name.split("(")[0].replace("void ", ""))
    return out


def test_dispatch_of_each_workload():
    g = lrgen.make(1)
    a, b = dev(g.t("a")), dev(g.t("b"))
    assert kernels(lambda: lr.lr_diag_scan(a, b)) == ["lr::diag_scan_narrow_kernel<float, 8, 512>"]

    g = lrgen.make(2, L=256)    # the headline's channels and batch; L does not pick the kernel
    T = {k: dev(g.t(k)) for k in ("x", "dt", "A", "B", "C", "Dskip")}
    assert kernels(lambda: lr.lr_selective_scan(T["x"], T["dt"], T["A"], T["B"], T["C"],
                                                T["Dskip"])) == \
        ["lr::selective_pair_kernel<unsigned short, 0, 64, 4, true>"]

    g = lrgen.make(3)
    T = {k: dev(g.t(k)) for k in ("x", "dt", "A", "B", "C", "Dskip")}
    assert kernels(lambda: lr.lr_ssd_scan(T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"],
                                          chunk=256)) == \
        ["lr::chunk_fwd_kernel<0, 128, false>"]   # 256 workgroups fill the chip: no split

    g = lrgen.make(4)
    T = {k: dev(g.t(k)) for k in ("q", "k", "v", "g")}
    assert kernels(lambda: lr.lr_gla_scan(T["q"], T["k"], T["v"], T["g"])) == \
        ["lr::chunk_fwd_kernel<2, 128, false>"]

    g = lrgen.make(5)
    T = {k: dev(g.t(k)) for k in ("x", "dt", "A", "B", "C", "Dskip", "dy")}
    ck = [None]

    def fwd():
        ck[0] = lr.lr_ssd_scan(T["x"], T["dt"], T["A"], T["B"], T["C"], T["Dskip"], chunk=256,
                               seg=256)[2]
    # 128 workgroups: the sequence is split, pre-pass then main pass
    assert kernels(fwd) == ["lr::chunk_fwd_kernel<0, 128, true>",
                            "lr::chunk_fwd_kernel<0, 128, false>"]
    assert kernels(lambda: lr.lr_ssd_scan_bwd(T["x"], T["dt"], T["A"], T["B"], T["C"],
                                              T["Dskip"], None, ck[0], T["dy"], chunk=256,
                                              seg=256)) == \
        ["lr::ssd_bwd_gloc_kernel<0, 128>", "lr::ssd_bwd_gcombine_kernel<0>",
         "lr::ssd_bwd_main_kernel<0, 128, 4>"] + \
        3 * ["lr::ssd_bwd_gloc_reduce_kernel<0, 128>", "lr::ssd_bwd_gcombine_kernel<0>",
             "lr::ssd_bwd_main_kernel<0, 128, 4>"] + \
        ["lr::ssd_bwd_reduce_kernel", "lr::ssd_bwd_reduce_kernel"]
    # one batch row per slice; each later slice's gloc runs beside the previous
    # slice's dB, dC reduction; the last slice's reduction, then dA, dD
