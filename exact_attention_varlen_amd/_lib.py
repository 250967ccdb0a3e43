"""ctypes loader for ``libattn_varlen.so`` (the gfx950 C ABI).

The library is built ahead of time by ``exact_attention_varlen_amd.build``. A
missing library is an error: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# ATTN_VARLEN_LIBRARY names another build of the same library in this directory
# (a variant built with `build.py --out NAME --extra -D...`, for comparisons)
_LIB_FILE = os.environ.get("ATTN_VARLEN_LIBRARY", "libattn_varlen.so")
if os.path.basename(_LIB_FILE) != _LIB_FILE or not _LIB_FILE.endswith(".so"):
    raise ValueError("ATTN_VARLEN_LIBRARY must name a .so file in the package directory")
LIB_PATH = os.path.join(HERE, _LIB_FILE)

_lock = threading.Lock()
_lib = None

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_f32 = ctypes.c_float
c_vp = ctypes.c_void_p
c_size = ctypes.c_size_t

_SIGNATURES = {
    "attn_varlen_fwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32,
                                       c_i32, c_f32, c_i32, c_vp, c_vp, c_vp]),
    "attn_varlen_fwd_window": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32,
                                              c_i32, c_i32, c_f32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "attn_varlen_bwd_window": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32,
                                              c_i32, c_i32, c_f32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                              c_vp, c_vp, c_size, c_vp]),
    "attn_varlen_fwd_splitkv": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32,
                                               c_i32, c_i32, c_i32, c_f32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp,
                                               c_vp, c_size, c_vp]),
    "attn_varlen_fwd_splitkv_workspace_size": (c_size, [c_i64, c_i32, c_i32, c_i32]),
    "attn_varlen_fwd_persistent": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32,
                                                  c_i32, c_i32, c_i32, c_f32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                                  c_vp]),
    "attn_varlen_fwd_num_splits": (c_i32, [c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "attn_varlen_bwd_workspace_size": (c_size, [c_i32, c_i64, c_i64, c_i32, c_i32, c_i32]),
    "attn_varlen_bwd_ds_workspace_size": (c_size, [c_i32, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "attn_varlen_bwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32,
                                       c_i32, c_f32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "attn_varlen_bwd_stored_ds": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32,
                                                 c_i32, c_i32, c_i32, c_f32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                                 c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "attn_varlen_bwd_noalloc": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32,
                                               c_i32, c_i32, c_f32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                               c_vp]),
    "attn_varlen_validate_seqlens": (ctypes.c_int, [c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp]),
    "attn_varlen_error_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_varlen_version": (ctypes.c_int, []),
    "attn_varlen_schedule_host": (c_i64, [c_vp, c_i32, c_i32, c_vp, c_vp, c_i64]),
    "attn_varlen_schedule_device": (ctypes.c_int, [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_i32, c_vp]),
    "attn_varlen_tile_plan_host": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "attn_varlen_exp2_fma_host": (ctypes.c_int, [c_vp, c_vp, c_i64]),
    "attn_varlen_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "attn_varlen_profile_count": (ctypes.c_int, []),
    "attn_varlen_profile_get": (ctypes.c_int, [ctypes.c_int, ctypes.c_char_p, ctypes.c_int, ctypes.POINTER(c_f32)]),
}


class LibraryMissing(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises LibraryMissing if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise LibraryMissing(
                    f"{LIB_PATH} is missing: build it with `python -m exact_attention_varlen_amd.build` "
                    "(there is no non-HIP fallback)")
            l = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(l, name)
                fn.restype = res
                fn.argtypes = args
            _lib = l
    return _lib


def exported_names():
    return list(_SIGNATURES)
