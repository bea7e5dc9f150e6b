"""Build liblr.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Usage:  python -m ssm_selective_scan_amd.build      (or build() from Python)
Objects go to ssm_selective_scan_amd/_build/, the library to
ssm_selective_scan_amd/liblr.so.  Every call recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
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


# Per-kernel register, scratch and LDS use, from the compiler's
# kernel-resource-usage remarks (the device code of the normal build; the
# objects go to _build/resources/ and are not linked).
RESOURCES = os.path.join(BUILD, "resources")
_REMARK_KEYS = {"VGPRs": "vgpr", "AGPRs": "agpr", "VGPRs Spill": "vgpr_spill",
                "SGPRs Spill": "sgpr_spill", "ScratchSize [bytes/lane]": "scratch",
                "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}


def _demangle(names):
    try:
        p = subprocess.run(["c++filt"], input="\n".join(names), stdout=subprocess.PIPE,
                           text=True, check=True)
        out = p.stdout.split("\n")[:len(names)]
    except (OSError, subprocess.CalledProcessError):
        return list(names)
    return [re.sub(r"^void ", "", re.sub(r"\(.*$", "", d)) for d in out]


def resource_usage(sources=None) -> list:
    """One dict per kernel of the given sources (default: all): name
    (demangled, without its parameter list), source, and the integers vgpr,
    agpr, vgpr_spill, sgpr_spill, scratch (bytes per lane), occupancy (waves
    per SIMD) and lds (bytes per workgroup, static)."""
    os.makedirs(RESOURCES, exist_ok=True)
    sources = list(sources or SOURCES)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        outs = list(ex.map(lambda s: _run([HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage",
                                           "-c", os.path.join(CSRC, s), "-o",
                                           os.path.join(RESOURCES, s.replace(".hip", ".o"))]),
                           sources))
    rows = []
    for src, out in zip(sources, outs):
        cur = None
        for line in out.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = {"name": m.group(1), "source": src}
                rows.append(cur)
                continue
            m = re.search(r"remark:\s+(.+?): (-?\d+) \[-Rpass-analysis", line)
            if m and cur is not None and m.group(1).strip() in _REMARK_KEYS:
                cur[_REMARK_KEYS[m.group(1).strip()]] = int(m.group(2))
    for r, d in zip(rows, _demangle([r["name"] for r in rows])):
        r["name"] = d
    return rows


if __name__ == "__main__":
    if "hostcheck" in sys.argv:
        print(build_hostcheck())
    elif "resources" in sys.argv:
        # python -m ssm_selective_scan_amd.build resources [file.hip ...]
        srcs = [a for a in sys.argv[1:] if a.endswith(".hip")]
        print(f"{'kernel':68s} {'VGPR':>4s} {'AGPR':>4s} {'spill':>5s} {'scratch':>7s} "
              f"{'waves':>5s} {'LDS':>7s}")
        for r in sorted(resource_usage(srcs or None), key=lambda r: r["name"]):
            print(f"{r['name'][:68]:68s} {r.get('vgpr', 0):4d} {r.get('agpr', 0):4d} "
                  f"{r.get('vgpr_spill', 0):5d} {r.get('scratch', 0):7d} "
                  f"{r.get('occupancy', 0):5d} {r.get('lds', 0):7d}")
    else:
        print(build(verbose="-v" in sys.argv))
