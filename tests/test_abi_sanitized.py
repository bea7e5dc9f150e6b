"""The C ABI's argument validation under AddressSanitizer and UBSan (CPU
only): every source is compiled host-only with both sanitizers, and every
check of test_abi.py runs against that library in a child process that
preloads the ASan runtime.  An out-of-bounds access, an overflow in a size
computation or any other undefined behaviour in the host code aborts the
child with a sanitizer report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import importlib.util, inspect, os, sys, types
root = sys.argv[1]
spec = importlib.util.spec_from_file_location(
    "ssm_selective_scan_amd._lib", os.path.join(root, "ssm_selective_scan_amd", "_lib.py"))
lib_mod = importlib.util.module_from_spec(spec)
spec.loader.exec_module(lib_mod)
lib_mod.LIB_PATH = sys.argv[2]
pkg = types.ModuleType("ssm_selective_scan_amd")
pkg._lib = lib_mod
sys.modules["ssm_selective_scan_amd"] = pkg
sys.modules["ssm_selective_scan_amd._lib"] = lib_mod
sys.path.insert(0, os.path.join(root, "tests"))
import test_abi
L = lib_mod.lib()
n = 0
for name, fn in inspect.getmembers(test_abi, inspect.isfunction):
    if name.startswith("test_"):
        fn(L)
        n += 1
print(f"sanitized ABI checks passed: {n}", flush=True)
"""


def test_abi_validation_under_asan_and_ubsan():
    from ssm_selective_scan_amd.build import asan_runtime, build_hostcheck
    lib = build_hostcheck()
    env = dict(os.environ, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([sys.executable, "-c", CHILD, ROOT, lib], env=env, capture_output=True,
                       text=True, timeout=300)
    out = p.stdout + p.stderr
    print(out[-3000:])
    assert p.returncode == 0, out[-3000:]
    assert "sanitized ABI checks passed" in p.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out
