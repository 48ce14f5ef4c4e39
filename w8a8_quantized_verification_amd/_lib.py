"""ctypes loader for libw8a8.so (argument marshalling only).

torch is imported first on purpose: it loads its bundled HIP runtime, and
libw8a8.so, whose dependency carries the same soname, then binds to that one
runtime, so device pointers and streams from torch are valid inside the
library.  There is no fallback: if the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch  # noqa: F401  (see module docstring)

PKG = os.path.dirname(os.path.abspath(__file__))
# W8A8_LIBRARY names another build of the same library (the sanitizer test
# loads a host-instrumented one this way); by default the in-tree build
LIB_PATH = os.environ.get("W8A8_LIBRARY") or os.path.join(PKG, "libw8a8.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "w8a8.h")

_c = ctypes
_i64, _sz, _vp, _i32 = _c.c_int64, _c.c_size_t, _c.c_void_p, _c.c_int32

# name -> (restype, argtypes); pointers are passed as integers (c_void_p)
SIGNATURES = {
    "w8a8_abi_version": (_i32, []),
    "w8a8_status_string": (_c.c_char_p, [_i32]),
    "w8a8_last_error": (_c.c_char_p, []),
    "w8a8_quantize_act": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_quantize_weight": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_tiled_weight_bytes": (_sz, [_i64, _i64]),
    "w8a8_quantize_weight_tiled": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_tile_weight": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "w8a8_linear_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "w8a8_linear_tiled": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "w8a8_linear": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "w8a8_verify_accept_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "w8a8_verify_accept": (_i32, [_vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "w8a8_lm_head_verify_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "w8a8_lm_head_verify": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp,
                                   _vp, _vp, _sz, _vp]),
    "w8a8_lm_head_verify_noalloc": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp,
                                           _vp, _vp, _vp, _vp]),
    "w8a8_lm_head_argmax": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "w8a8_accept_from_keys": (_i32, [_vp, _sz, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "w8a8_lm_head_argmax_tiled_act": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _sz,
                                             _vp]),
    "w8a8_lm_head_argmax_timed": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _sz, _vp,
                                         _vp, _vp]),
    "w8a8_hbm_read_probe": (_i32, [_vp, _sz, _vp, _vp, _vp, _vp]),
    "w8a8_bf16_linear": (_i32, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_bf16_tiled_weight_bytes": (_sz, [_i64, _i64]),
    "w8a8_tile_weight_bf16": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "w8a8_bf16_linear_tiled": (_i32, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_verify_sample_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "w8a8_verify_sample": (_i32, [_vp, _i64, _vp, _i64, _i64, _c.c_float, _vp, _vp, _vp, _vp,
                                  _vp, _sz, _vp]),
    "w8a8_sample_weights_workspace_bytes": (_sz, [_i64, _i64]),
    "w8a8_sample_weights": (_i32, [_vp, _i64, _i64, _c.c_float, _vp, _vp, _sz, _vp]),
    "w8a8_w4_weight_bytes": (_sz, [_i64, _i64]),
    "w8a8_quantize_weight_w4": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_linear_w4": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "w8a8_lm_head_argmax_w4": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "w8a8_residual_rmsnorm_quant": (_i32, [_vp, _vp, _vp, _c.c_float, _vp, _i64, _i64, _vp, _vp,
                                           _vp, _vp, _vp]),
    "w8a8_silu_mul_quant": (_i32, [_vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "w8a8_quantize_act_tiled": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_linear_tiled_act_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "w8a8_linear_tiled_act": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz,
                                     _vp]),
    "w8a8_verify_attention_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "w8a8_pack_v_cache": (_i32, [_vp, _i64, _i64, _i64, _i64, _vp, _vp]),
    "w8a8_qk_norm_rope_append": (_i32, [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _c.c_float,
                                        _c.c_float, _vp, _i64, _vp, _vp, _vp, _vp]),
    "w8a8_verify_attention": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp,
                                     _vp, _sz, _vp]),
}

_lib = None


class W8A8Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def header_functions(path: str = HEADER) -> list:
    """Names of the functions include/w8a8.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m w8a8_quantized_verification_amd.build` "
                "(the W8A8 path has no CPU fallback)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(status: int) -> None:
    if status != 0:
        l = lib()
        msg = l.w8a8_last_error().decode() or l.w8a8_status_string(status).decode()
        raise W8A8Error(status, msg)
