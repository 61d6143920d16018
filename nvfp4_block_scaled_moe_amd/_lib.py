"""ctypes loader for libnvfp4moe.so: the exact C ABI of include/nvfp4moe.h.

The shared library must have been built in-tree (``__graft_entry__.build()`` or
``python nvfp4_block_scaled_moe_amd/build.py``). There is no fallback: if the library is
missing or lacks a symbol, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.environ.get("NVFP4MOE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libnvfp4moe.so")

# enums (include/nvfp4moe.h)
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
W4A16, W4A4, W4A16_PREPARED = 0, 1, 2
EPI_NONE, EPI_SWIGLU = 0, 1
F32, BF16 = 0, 1
LAYOUT_ROW_MAJOR, LAYOUT_TILED = 0, 1
PATH_NONE, PATH_STREAM, PATH_MFMA = 0, 1, 2
STATUS_NAMES = {0: "OK", 1: "ERR_INVALID_ARG", 2: "ERR_UNSUPPORTED", 3: "ERR_WORKSPACE", 4: "ERR_HIP"}

_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
_int = ctypes.c_int

#: name -> (restype, argtypes), one entry per function declared in include/nvfp4moe.h
SIGNATURES = {
    "nvfp4_quantize": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp, _int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_quantize_workspace_size": (_sz, [_i64, _i64, _i64]),
    "nvfp4_quantize_noalloc": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp, _int, _vp, _vp, _vp, _vp]),
    "nvfp4_weights_tile": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "nvfp4_tiled_codes_bytes": (_sz, [_i64, _i64]),
    "nvfp4_tiled_scales_bytes": (_sz, [_i64, _i64]),
    "moe_route_permute": (_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_route_permute_workspace_size": (_sz, [_i32, _i32, _i32]),
    "moe_dispatch_w4a16": (_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _sz, _vp]),
    "moe_dispatch_w4a16_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "moe_prepared_act_bytes": (_sz, [_i64, _i32]),
    "moe_grouped_gemm_nvfp4": (_int, [_int, _int, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _int, _vp, _vp,
                                      _sz, _vp]),
    "moe_grouped_gemm_workspace_size": (_sz, [_int, _i64, _i32, _i32, _i32, _i32]),
    "moe_grouped_gemm_nvfp4_combine": (_int, [_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _i32, _i32, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm_nvfp4_combine_workspace_size": (_sz, [_int, _i32, _i32, _i32, _i32, _i32]),
    "moe_grouped_gemm_mxfp4_combine": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                              _i32, _i32, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm_mxfp4_combine_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "moe_unpermute_reduce": (_int, [_vp, _int, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "act_fp8_e4m3_roundtrip": (_int, [_vp, _i64, _vp, _vp, _sz, _vp]),
    "act_fp8_e4m3_roundtrip_workspace_size": (_sz, [_i64]),
    "mxfp4_quantize": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp]),
    "mxfp4_tiled_scales_bytes": (_sz, [_i64, _i64]),
    "mxfp4_weights_tile": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "moe_grouped_gemm_mxfp4": (_int, [_int, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                      _i32, _i32, _vp, _int, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm_mxfp4_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "moe_grouped_gemm_mxfp4_swiglu_q": (_int, [_vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                               _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "mxfp8_quantize": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp]),
    "mxfp8_tiled_codes_bytes": (_sz, [_i64, _i64]),
    "mxfp8_weights_tile": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "moe_grouped_gemm_mxfp8": (_int, [_int, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                      _i32, _i32, _vp, _int, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm_mxfp8_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "nvfp4moe_last_error": (ctypes.c_char_p, []),
    "nvfp4moe_last_dispatch": (_int, []),
    "nvfp4moe_abi_version": (_int, []),
}

_lock = threading.Lock()
_lib = None


class NVFP4MoEError(RuntimeError):
    def __init__(self, fn, status, message):
        super().__init__(f"{fn} failed with {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load (once) and return the ctypes library with every signature declared."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise ImportError(f"{path} is not built; run __graft_entry__.build() first")
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)      # AttributeError if a symbol is missing
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def check(fn_name: str, status: int):
    if status != OK:
        msg = load().nvfp4moe_last_error().decode(errors="replace")
        raise NVFP4MoEError(fn_name, status, msg)
