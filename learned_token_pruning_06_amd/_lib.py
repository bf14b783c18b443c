"""ctypes loader of libtokengate.so and the prototypes of its C ABI.

There is no fallback: if the library is missing or does not load, every
call raises.  torch is imported first when present so that the library binds
to the same HIP runtime as torch (both carry the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("TG_LIBRARY", os.path.join(_PKG, "libtokengate.so"))

TG_OK, TG_ERR_INVALID_ARG, TG_ERR_UNSUPPORTED, TG_ERR_WORKSPACE, TG_ERR_HIP = range(5)
TG_F32, TG_BF16 = 0, 1
CONTRACT_BITS = {"offsets": 0x1, "negative_budget": 0x2, "capacity": 0x4, "index": 0x8,
                 "kept_offsets": 0x10, "positions": 0x20}

c_vp, c_i32, c_i64, c_f32, c_sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_float, ctypes.c_size_t)

# name -> (restype, argtypes); the exported symbols of include/tokengate.h
PROTOTYPES = {
    "tg_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tg_last_error": (ctypes.c_char_p, []),
    "tg_version": (ctypes.c_int, []),
    "tg_score_workspace_size": (c_sz, [c_i64, c_i32]),
    "tg_score": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp,
                                c_f32, c_vp, c_vp, c_i32, c_f32, c_f32, c_vp, c_vp, c_vp, c_sz,
                                c_vp]),
    "tg_kept_sizes": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp]),
    "tg_select_workspace_size": (c_sz, [c_i64, c_i32]),
    "tg_select_topk": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_vp, c_vp,
                                      c_vp, c_vp, c_vp, c_sz, c_vp]),
    "tg_select_topk_noalloc": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_vp,
                                              c_vp, c_vp, c_vp, c_vp]),
    "tg_gather": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "tg_qkv_proj": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i32, c_vp, c_i32, c_i32,
                                   c_i32, c_vp, c_vp, c_vp, c_vp]),
    "tg_qkv_proj_rope": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i32, c_vp, c_i32,
                                        c_i32, c_i32, c_vp, c_vp, c_vp, c_f32, c_f32, c_vp, c_vp,
                                        c_vp, c_vp]),
    "tg_gated_attn": (ctypes.c_int, [c_vp, c_vp, c_vp, ctypes.c_int, c_vp, c_i64, c_vp, c_vp,
                                     c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_f32,
                                     c_vp, c_vp]),
    "tg_gated_attn_split_workspace_size": (c_sz, [c_i64, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "tg_gated_attn_split": (ctypes.c_int, [c_vp, c_vp, c_vp, ctypes.c_int, c_vp, c_i64, c_vp,
                                           c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp,
                                           c_vp, c_f32, c_vp, c_vp, c_sz, c_vp]),
    "tg_score_bwd_workspace_size": (c_sz, [c_i64, c_i32, c_i32, c_i32]),
    "tg_score_bwd": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp,
                                    c_vp, c_vp, c_vp, c_i32, c_f32, c_f32, c_vp, c_vp, c_vp, c_i64,
                                    c_vp,
                                    c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "tg_gated_attn_bwd_workspace_size": (c_sz, [c_i64, c_i32, c_i32, c_i32]),
    "tg_gated_attn_bwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, ctypes.c_int, c_i64, c_vp, c_vp,
                                         c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_f32,
                                         c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                         c_sz, c_vp]),
    "tg_set_contract_checks": (ctypes.c_int, [c_i32]),
    "tg_contract_status": (ctypes.c_int, [c_vp, c_vp]),
    "tg_gated_decode_workspace_size": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i64]),
    "tg_gated_decode": (ctypes.c_int, [c_vp, c_vp, c_vp, ctypes.c_int, c_vp, c_i64, c_vp, c_vp,
                                       c_vp, c_i32, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp,
                                       c_f32, c_vp, c_sz, c_vp]),
}

_lock = threading.Lock()
_lib = None


class TokenGateError(RuntimeError):
    def __init__(self, fn: str, status: int, lib):
        self.status = status
        name = lib.tg_status_string(status).decode()
        detail = lib.tg_last_error().decode()
        super().__init__(f"{fn} failed: {name}: {detail}")


def load():
    """Load libtokengate.so once; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libtokengate.so not found at {LIB_PATH}; build it with "
                "`python -m learned_token_pruning_06_amd.build` (no CPU fallback exists)")
        try:
            import torch  # noqa: F401  -- share torch's HIP runtime
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(fn: str, status: int):
    if status != TG_OK:
        raise TokenGateError(fn, status, load())
