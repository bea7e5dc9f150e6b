"""Build liblr.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Usage:  python -m ssm_selective_scan_amd.build      (or build() from Python)
Objects go to ssm_selective_scan_amd/_build/, the library to
ssm_selective_scan_amd/liblr.so.  Every call recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblr.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.hip", "diag_scan.hip", "selective_scan.hip", "selective_bwd.hip", "chunk_scan.hip",
           "ssd_bwd.hip", "step.hip", "rotlru.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast",
    # MFMA accumulators in ordinary VGPRs: no copies between AGPRs and VGPRs
    # where an accumulator is also an operand or is scaled by VALU code
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

# hipcc's host pass does not know the device feature above; the warning is harmless.
_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if _NOISE not in l)
    if p.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(BUILD, s.replace(".hip", ".o"))
            objs.append(obj)
            jobs.append(ex.submit(_run, [HIPCC, *FLAGS, "-c", src, "-o", obj]))
        for j in jobs:
            out = j.result()
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


# A build whose host code carries AddressSanitizer and UBSan (the device
# code is compiled as usual, without them), for the CPU tests of the C ABI's
# argument validation.
HOSTCHECK = os.path.join(BUILD, "hostcheck")
HOSTCHECK_LIB = os.path.join(HOSTCHECK, "liblr_hostcheck.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang ASan runtime matching hipcc, to preload into the process
    that loads the sanitized library."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return hits[-1]


def build_hostcheck() -> str:
    os.makedirs(HOSTCHECK, exist_ok=True)
    objs, jobs = [], []
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for s in SOURCES:
            obj = os.path.join(HOSTCHECK, s.replace(".hip", ".o"))
            objs.append(obj)
            jobs.append(ex.submit(_run, [HIPCC, *FLAGS, *SAN, "-c", os.path.join(CSRC, s),
                                         "-o", obj]))
        for j in jobs:
            j.result()
    tmp = HOSTCHECK_LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-Xarch_host",
          "-shared-libasan", "-o", tmp, *objs])
    os.replace(tmp, HOSTCHECK_LIB)
    return HOSTCHECK_LIB


if __name__ == "__main__":
    if "hostcheck" in sys.argv:
        print(build_hostcheck())
    else:
        print(build(verbose="-v" in sys.argv))
