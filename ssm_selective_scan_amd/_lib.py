"""ctypes loader for liblr.so and the raw C signatures of include/lr.h.

There is no fallback: if the library is missing or fails to load, importing
the functions raises.  Build it with ``python -m ssm_selective_scan_amd.build``.
"""
from __future__ import annotations

import ctypes as C
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblr.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "lr.h")

LR_F32, LR_BF16 = 0, 1
LR_DISC_ZOH, LR_DISC_EULER, LR_DISC_BILINEAR, LR_DISC_DIRAC = 0, 1, 2, 3
STATUS = {0: "LR_OK", 1: "LR_E_NULLPTR", 2: "LR_E_SHAPE", 3: "LR_E_DTYPE", 4: "LR_E_ALIGN",
          5: "LR_E_UNSUPPORTED", 6: "LR_E_WORKSPACE", 7: "LR_E_OVERFLOW", 8: "LR_E_HIP"}

_i64, _p, _f32p, _int, _sz = C.c_int64, C.c_void_p, C.c_void_p, C.c_int, C.c_size_t

SIGNATURES = {
    "lr_status_string": (C.c_char_p, [_int]),
    "lr_version": (C.c_char_p, []),
    "lr_diag_scan": (_int, [_int, _i64, _i64, _i64, _p, _p, _f32p, _p, _f32p, _p]),
    "lr_diag_scan_bwd": (_int, [_int, _i64, _i64, _i64, _p, _p, _f32p, _p, _f32p, _p, _p, _f32p,
                                _p]),
    "lr_selective_scan": (_int, [_int, _int, _i64, _i64, _i64, _i64, _i64, _p, _p, _f32p, _p,
                                 _p, _f32p, _f32p, _p, _f32p, _f32p, _p]),
    "lr_selective_scan_bwd_workspace_bytes": (_sz, [_i64] * 5),
    "lr_selective_scan_bwd": (_int, [_int, _int] + [_i64] * 5 + [_p, _p, _f32p, _p, _p, _f32p,
                                                                 _f32p, _p, _f32p, _p, _p, _f32p,
                                                                 _p, _p, _f32p, _f32p, _p, _sz,
                                                                 _p]),
    "lr_ssd_scan": (_int, [_int, _int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p,
                           _f32p, _p, _p, _f32p, _f32p, _p, _f32p, _f32p, _p, _sz, _p]),
    "lr_ssd_scan_workspace_bytes": (_sz, [_i64] * 7),
    "lr_ssd_scan_noalloc": (_int, [_int, _int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                   _p, _p, _f32p, _p, _p, _f32p, _f32p, _p, _f32p, _f32p, _p]),
    "lr_ssd_scan_bwd_workspace_bytes": (_sz, [_i64] * 8),
    "lr_ssd_scan_bwd": (_int, [_int, _int] + [_i64] * 8 + [_p, _p, _f32p, _p, _p, _f32p, _f32p,
                                                            _f32p, _p, _f32p, _p, _p, _f32p, _p,
                                                            _p, _f32p, _f32p, _p, _sz, _p]),
    "lr_gla_scan": (_int, [_int] + [_i64] * 7 + [_p, _p, _p, _p, _f32p, _p, _f32p, _f32p, _p, _sz,
                                                 _p]),
    "lr_gla_scan_workspace_bytes": (_sz, [_i64] * 6),
    "lr_gla_scan_bwd_workspace_bytes": (_sz, [_i64] * 7),
    "lr_gla_scan_bwd": (_int, [_int] + [_i64] * 7 + [_p, _p, _p, _p, _f32p, _p, _f32p, _p, _p, _p,
                                                     _p, _f32p, _p, _sz, _p]),
    "lr_rotlru_scan": (_int, [_int, _i64, _i64, _i64, _p, _p, _p, _f32p, _p, _f32p, _p]),
    "lr_rotlru_scan_bwd": (_int, [_int, _i64, _i64, _i64, _p, _p, _p, _f32p, _p, _f32p, _p, _p,
                                  _p, _f32p, _p]),
    "lr_diag_step": (_int, [_int, _i64, _i64, _p, _p, _f32p, _p, _p]),
    "lr_selective_step": (_int, [_int, _int, _i64, _i64, _i64, _p, _p, _f32p, _p, _p, _f32p,
                                 _f32p, _p, _p]),
    "lr_ssd_step": (_int, [_int, _int] + [_i64] * 5 + [_p, _p, _f32p, _p, _p, _f32p, _f32p, _p,
                                                       _p]),
    "lr_gla_step": (_int, [_int] + [_i64] * 4 + [_p, _p, _p, _p, _f32p, _p, _p]),
}


def header_symbols() -> list:
    """Names of the functions declared in include/lr.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(lr_\w+)\s*\(", text, re.M)))


_LIB = None


def lib() -> C.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"liblr.so not found at {LIB_PATH}; build it with "
                               "`python -m ssm_selective_scan_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


class LrError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = lib().lr_status_string(code).decode()
        super().__init__(f"{fn} failed with {STATUS.get(code, code)}: {msg}")


def check(fn: str, code: int) -> None:
    if code != 0:
        raise LrError(fn, code)
