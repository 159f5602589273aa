"""ctypes view of libsgemm.so (the C ABI in include/sgemm.h, window_sum.h,
conv2d.h and attention.h).

Argument marshalling only: every operation runs in the HIP library.  If the
library has not been built, loading fails with an error that says so; there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsgemm.so")
# Test library: the same C ABI built with SGEMM_RACECHECK=1 (LDS buffers
# filled with NaN once consumed, tiles in reverse order).
RACECHECK_LIB_PATH = os.path.join(PKG, "libsgemm_racecheck.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HEADER = os.path.join(INCLUDE, "sgemm.h")

STATUS = {
    0: "SGEMM_STATUS_SUCCESS",
    -1: "SGEMM_STATUS_INVALID_SIZE",
    -2: "SGEMM_STATUS_INVALID_LD",
    -3: "SGEMM_STATUS_NULL_POINTER",
    -4: "SGEMM_STATUS_SIZE_OVERFLOW",
    -5: "SGEMM_STATUS_INVALID_STRIDE",
    -6: "SGEMM_STATUS_LAUNCH_FAILED",
    -7: "SGEMM_STATUS_INVALID_CONFIG",
    -8: "SGEMM_STATUS_INVALID_OP",
}


class SgemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, status_string(status), status))


_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_SIGS = {
    "sgemm": ([_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p], ctypes.c_int),
    "sgemm_valu": ([_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p], ctypes.c_int),
    "sgemm_strided_batched": (
        [_i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _p],
        ctypes.c_int),
    "sgemm_valu_strided_batched": (
        [_i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _p],
        ctypes.c_int),
    "sgemm_with_config": (
        [ctypes.c_int, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64,
         _p], ctypes.c_int),
    "sgemm_num_configs": ([], ctypes.c_int),
    "sgemm_config_info": ([ctypes.c_int, ctypes.c_char_p, _i64, ctypes.POINTER(ctypes.c_int),
                           ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                           ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
    "sgemm_select_config": ([_i64, _i64, _i64, _i64], ctypes.c_int),
    "sgemm_config_selectable": ([ctypes.c_int], ctypes.c_int),
    "sgemm_config_workgroups_per_cu": ([ctypes.c_int], ctypes.c_int),
    "sgemm_ex": ([ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, ctypes.c_float, _p, _i64, _p,
                  _i64, ctypes.c_float, _p, _i64, _p], ctypes.c_int),
    "sgemm_ex_strided_batched": (
        [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, ctypes.c_float, _p, _i64, _i64, _p, _i64,
         _i64, ctypes.c_float, _p, _i64, _i64, _i64, _p], ctypes.c_int),
    "sgemm_ex_with_config": (
        [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, ctypes.c_float, _p, _i64,
         _i64, _p, _i64, _i64, ctypes.c_float, _p, _i64, _i64, _i64, _p], ctypes.c_int),
    "sgemm_config_has_general_form": ([ctypes.c_int], ctypes.c_int),
    "sgemm_select_general_config": ([_i64, _i64, _i64, _i64], ctypes.c_int),
    "sgemm_config_predict_us": ([ctypes.c_int, _i64, _i64, _i64, _i64], ctypes.c_double),
    "sgemm_autotune": (
        [_i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _p,
         ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float)],
        ctypes.c_int),
    "sgemm_splitk": ([ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _p,
                      _i64, _p], ctypes.c_int),
    "sgemm_splitk_noalloc": ([ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64,
                              _i64, _p], ctypes.c_int),
    "sgemm_splitk_plan": ([ctypes.c_int, _i64, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_int),
                           ctypes.POINTER(_i64)], _i64),
    "sgemm_splitk_plan_full_tiles": ([ctypes.c_int, _i64, _i64, _i64, _i64], _i64),
    "sgemm_config_has_splitk": ([ctypes.c_int], ctypes.c_int),
    "sgemm_ex_splitk": ([ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64, _i64,
                         ctypes.c_float, _p, _i64, _p, _i64, ctypes.c_float, _p, _i64, _i64, _p,
                         _i64, _p], ctypes.c_int),
    "sgemm_ex_splitk_plan": ([ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _i64,
                              ctypes.POINTER(ctypes.c_int), ctypes.POINTER(_i64)], _i64),
    "sgemm_ex_splitk_plan_full_tiles": ([ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64,
                                         _i64, _i64], _i64),
    "sgemm_config_has_general_splitk": ([ctypes.c_int], ctypes.c_int),
    "sgemm_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "window_sum": ([_i64, _i64, _p, _p, _p], ctypes.c_int),
    "conv2d_nhwc": ([_i64] * 13 + [_p, _p, _p, _p], ctypes.c_int),
    "conv2d_nhwc_with_config": ([ctypes.c_int] + [_i64] * 13 + [_p, _p, _p, _p], ctypes.c_int),
    "conv2d_nhwc_output_size": ([_i64] * 10 + [ctypes.POINTER(_i64), ctypes.POINTER(_i64)],
                                ctypes.c_int),
    "conv2d_config_available": ([ctypes.c_int], ctypes.c_int),
    "conv2d_select_config": ([_i64] * 13, ctypes.c_int),
    "conv2d_nhwc_splitk": ([ctypes.c_int] + [_i64] * 13 + [_p, _p, _p, _i64, _p, _i64, _p],
                           ctypes.c_int),
    "conv2d_nhwc_splitk_plan": ([ctypes.c_int] + [_i64] * 14 +
                                [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(_i64),
                                 ctypes.POINTER(_i64)], _i64),
    "conv2d_config_has_splitk": ([ctypes.c_int], ctypes.c_int),
    "attention_fwd": ([_i64, _i64, _i64, _i64, _p, _p, _p, _p, ctypes.c_float, ctypes.c_int, _p],
                      ctypes.c_int),
}


_racecheck_lib = None


def _load(path: str):
    if not os.path.exists(path):
        raise RuntimeError(
            "%s is not built (%s); run `python -m tiled_fp32_gemm_sgemm_amd.build`"
            % (os.path.basename(path), path))
    handle = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(handle, name)
        fn.argtypes = args
        fn.restype = res
    return handle


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def racecheck_lib():
    """The race-check build of the same C ABI (tests only); raises if it has
    not been built."""
    global _racecheck_lib
    if _racecheck_lib is None:
        _racecheck_lib = _load(RACECHECK_LIB_PATH)
    return _racecheck_lib


def status_string(status: int) -> str:
    return lib().sgemm_status_string(int(status)).decode()


def header_functions(path: str | None = None):
    """Names of the functions the headers under include/ declare (one header
    when `path` is given)."""
    paths = [path] if path else sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)
                                       if f.endswith(".h"))
    names = set()
    for p in paths:
        text = re.sub(r"/\*.*?\*/", " ", open(p).read(), flags=re.S)
        text = re.sub(r"#.*", " ", text)
        names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)
