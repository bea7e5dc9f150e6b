"""GPU parity of lr_rotlru_scan (complex-diagonal recurrence over channel
pairs) against the fp64 oracle, through the C ABI."""
import pytest
import torch

import lrgen
import oracle
import ssm_selective_scan_amd as lr
from gpu_util import TOL, check, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("B,L,D", [(1, 1024, 256), (2, 1500, 38), (1, 1, 2), (3, 513, 64),
                                   (1, 4097, 40)])
def test_rotlru_parity(io, B, L, D):
    print(f"rotlru io={io} B={B} L={L} D={D}", flush=True)
    g = lrgen.make(6, io=io, B=B, L=L, D=D)
    h0 = lrgen.state_normal((B, D), 6)
    h, hl = lr.lr_rotlru_scan(dev(g.t("r")), dev(g.t("theta")), dev(g.t("u")), h0=dev(h0),
                              want_last=True)
    torch.cuda.synchronize()
    ref, ref_last = oracle.rotlru_scan(g["r"], g["theta"], g["u"], h0)
    check("h", h, ref, TOL[io])
    check("h_last", hl, ref_last, TOL["f32"] if io == "f32" else TOL["bf16"])


def test_rotlru_empty_and_determinism():
    h0 = torch.randn(2, 6, device="cuda")
    z = torch.empty(2, 0, 3, device="cuda")
    _, hl = lr.lr_rotlru_scan(z, z, torch.empty(2, 0, 6, device="cuda"), h0=h0, want_last=True)
    torch.cuda.synchronize()
    assert torch.equal(hl, h0)
    g = lrgen.make(6)
    args = (dev(g.t("r")), dev(g.t("theta")), dev(g.t("u")))
    r1, _ = lr.lr_rotlru_scan(*args)
    r2, _ = lr.lr_rotlru_scan(*args)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)
