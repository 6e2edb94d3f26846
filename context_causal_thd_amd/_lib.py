"""ctypes loader for libcpthd.so (the in-tree C-ABI library).

There is no fallback: if the library is missing every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; CPTHD_LIB names another build of the same library (a variant built with
# `python -m context_causal_thd_amd.build --out <path> -D...`)
LIB_PATH = os.environ.get("CPTHD_LIB") or os.path.join(_HERE, "libcpthd.so")

c_i32, c_i64, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/cpthd.h and include/cpthd_timing.h
SIGNATURES = {
    "cpthd_partition_indices": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "cpthd_reorder_kv": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp]),
    "cpthd_gather_rows": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp]),
    "cpthd_attn_workspace_bytes": (c_sz, [c_i64, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "cpthd_attn_workspace_min_bytes": (c_sz, [c_i64, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "cpthd_attn_plan": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                c_vp, c_sz, c_vp, c_vp]),
    "cpthd_attn_fwd": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32,
                               c_i32, c_f32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp, c_vp]),
    "cpthd_attn_bwd": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32, c_i32,
                               c_i32, c_i32, c_i32, c_i32, c_f32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz,
                               c_vp, c_vp]),
    "cpthd_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}
# K/V in rank-major all-gathered order: same arguments as the physical-order calls
SIGNATURES["cpthd_attn_fwd_allgathered"] = SIGNATURES["cpthd_attn_fwd"]
SIGNATURES["cpthd_attn_bwd_allgathered"] = SIGNATURES["cpthd_attn_bwd"]
# allocation-free backward: cpthd_attn_bwd without the workspace pointer and size
SIGNATURES["cpthd_attn_bwd_noalloc"] = (c_i32, SIGNATURES["cpthd_attn_bwd"][1][:24] + [c_vp, c_vp])
# instrumentation variants (include/cpthd_timing.h): + kv_allgathered, events, n_events
SIGNATURES["cpthd_attn_fwd_timed"] = (c_i32, SIGNATURES["cpthd_attn_fwd"][1] + [c_i32, c_vp, c_i32])
SIGNATURES["cpthd_attn_bwd_timed"] = (c_i32, SIGNATURES["cpthd_attn_bwd"][1] + [c_i32, c_vp, c_i32])

_lib = None


def load():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m context_causal_thd_amd.build`")
        import torch  # noqa: F401  -- binds the library to the HIP runtime torch already loaded
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class CpthdError(RuntimeError):
    def __init__(self, fn, status):
        msg = load().cpthd_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def call(name, *args):
    status = getattr(load(), name)(*args)
    if status < 0:
        raise CpthdError(name, status)
    return status
