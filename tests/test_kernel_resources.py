"""Register, scratch and LDS use of the kernels the five workloads dispatch,
from the compiler's kernel-resource-usage remarks (a cross-compile for
gfx950; no GPU needed).  A kernel that starts to spill registers to scratch
memory, or whose occupancy drops, fails here before any timing shows it."""
import pytest

from ssm_selective_scan_amd import build

# kernel -> waves per SIMD the workload's launch relies on
HOT = {
    "lr::diag_scan_narrow_kernel<float, 8, 512>": 2,              # diagonal, B=1 L=1024 D=256
    "lr::selective_pair_kernel<unsigned short, 0, 64, 4, true>": 2,  # Mamba-1 ZOH (two workgroups per CU)
    "lr::chunk_fwd_kernel<0, 128, false>": 1,                      # SSD, and main pass with checkpoints
    "lr::chunk_fwd_kernel<0, 128, true>": 1,                       # SSD pre-pass of a split sequence
    "lr::chunk_fwd_kernel<2, 128, false>": 1,                      # GLA
    "lr::ssd_bwd_gloc_kernel<0, 128>": 1,                          # SSD backward launches
    "lr::ssd_bwd_gloc_reduce_kernel<0, 128>": 1,
    "lr::ssd_bwd_gcombine_kernel<0>": 1,
    "lr::ssd_bwd_main_kernel<0, 128, 4>": 1,
    "lr::ssd_bwd_reduce_kernel": 1,
}
LDS_PER_WORKGROUP = 160 * 1024   # gfx950


@pytest.fixture(scope="module")
def rows():
    return build.resource_usage(["diag_scan.hip", "selective_scan.hip", "chunk_scan.hip",
                                 "ssd_bwd.hip"])


def test_hot_kernels_keep_registers_and_occupancy(rows):
    by = {r["name"]: r for r in rows}
    for name, waves in HOT.items():
        assert name in by, f"{name} not compiled"
        r = by[name]
        assert r.get("vgpr_spill", 0) == 0 and r.get("scratch", 0) == 0, (name, r)
        assert r["occupancy"] >= waves, (name, r)


def test_static_lds_fits_a_workgroup(rows):
    assert rows
    for r in rows:
        assert r.get("lds", 0) <= LDS_PER_WORKGROUP, r
