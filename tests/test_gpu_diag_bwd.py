"""GPU parity of lr_diag_scan_bwd (reverse-time adjoint of the diagonal
recurrence) against the fp64 oracle, through the C ABI."""
import pytest
import torch

import lrgen
import oracle
import ssm_selective_scan_amd as lr
from gpu_util import TOL, check, dev

pytestmark = pytest.mark.gpu


def _round_io(x, io):
    return lrgen.round_bf16(x) if io == "bf16" else lrgen.round_f32(x)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("B,L,D", [(1, 1024, 256), (2, 1500, 37), (1, 1, 5), (3, 513, 16),
                                   (1, 4097, 20),
                                   # wide channel tiles: 4 and 2 channels per lane
                                   (64, 600, 512), (33, 130, 514)])
def test_diag_bwd_parity(io, B, L, D):
    print(f"diag bwd io={io} B={B} L={L} D={D}", flush=True)
    g = lrgen.make(1, io=io, B=B, L=L, D=D, grads=True)
    h0 = lrgen.state_normal((B, D), 1)
    dhl = lrgen.state_normal((B, D), 1, tensor_id=21)
    a = dev(g.t("a"))
    # both sides differentiate at the oracle's own forward states, rounded to
    # io as a forward output would be (the forward is checked on its own)
    hh = _round_io(oracle.diag_scan(g["a"], g["b"], h0)[0], io)
    da, db, dh0 = lr.lr_diag_scan_bwd(a, dev(hh, io), dev(g.t("dh")), h0=dev(h0),
                                      dh_last=dev(dhl), want_dh0=True)
    torch.cuda.synchronize()
    rda, rdb, rdh0 = oracle.diag_scan_bwd(g["a"], hh, g["dh"], h0, dhl)
    check("da", da, rda, TOL[io])
    check("db", db, rdb, TOL[io])
    check("dh0", dh0, rdh0, TOL["f32"] if io == "f32" else TOL["bf16"])


def test_diag_bwd_empty_and_determinism():
    dhl = torch.randn(2, 7, device="cuda")
    z = torch.empty(2, 0, 7, device="cuda")
    _, _, dh0 = lr.lr_diag_scan_bwd(z, z, z, dh_last=dhl, want_dh0=True)
    torch.cuda.synchronize()
    assert torch.equal(dh0, dhl)
    g = lrgen.make(1, grads=True)
    a, b, dh = dev(g.t("a")), dev(g.t("b")), dev(g.t("dh"))
    h, _ = lr.lr_diag_scan(a, b)
    r1 = lr.lr_diag_scan_bwd(a, h, dh)
    r2 = lr.lr_diag_scan_bwd(a, h, dh)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
