"""ctypes declarations of the C ABI in include/oscar.h.

Loads the in-tree ``libkv_cache_int2_amd.so``.  There is no fallback of any
kind: if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkv_cache_int2_amd.so")


class OscarShape(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("group_size", C.c_int32), ("page_size", C.c_int32), ("window", C.c_int32),
                ("n_sink", C.c_int32)]


P = C.c_void_p
I32, I64, SZ = C.c_int32, C.c_int64, C.c_size_t
SHAPE = C.POINTER(OscarShape)

# name -> (restype, argtypes); mirrors include/oscar.h
SIGNATURES = {
    "oscar_calibrate": (C.c_int, [SHAPE, P, I64, P, P, I64, P, P, P, P]),
    "oscar_calibrate_layers": (C.c_int, [SHAPE, I32, P, I64, P, P, I64, P, P, P, P]),
    "oscar_rotation_file_bytes": (SZ, [I32, I32, I32]),
    "oscar_rotation_write": (C.c_int, [C.c_char_p, SHAPE, I32, P, P, P, P]),
    "oscar_rotation_read_info": (C.c_int, [C.c_char_p, C.POINTER(I32), C.POINTER(I32), C.POINTER(I32),
                                           C.POINTER(I32)]),
    "oscar_rotation_read": (C.c_int, [C.c_char_p, SHAPE, I32, P, P, P, P]),
    "oscar_quantize_append": (C.c_int, [SHAPE, P, P, P, P, I64, P, P, I32, P, I32, P, P, I64, P, P, P]),
    "oscar_decode_workspace_bytes": (SZ, [SHAPE, I32, I32]),
    "oscar_quantize_append_layers": (C.c_int, [SHAPE, I32, P, P, P, P, I64, P, P, I32, P, I32, P, P, I64, P, P,
                                               P]),
    "oscar_decode_layers_workspace_bytes": (SZ, [SHAPE, I32, I32, I32]),
    "oscar_decode_attn_layers": (C.c_int, [SHAPE, I32, P, P, P, I32, P, I32, P, I32, P, I64, P, P, P, P, SZ, P]),
    "oscar_decode_attn": (C.c_int, [SHAPE, P, P, P, I32, P, I32, P, I32, P, I64, P, P, P, P, SZ, P]),
    "oscar_decode_noalloc_scratch_bytes": (SZ, [SHAPE, I32, I32]),
    "oscar_decode_attn_noalloc": (C.c_int, [SHAPE, P, P, P, I32, P, I32, P, I32, P, I64, P, P, P, P]),
    "oscar_bf16_append": (C.c_int, [SHAPE, P, P, I64, P, P, I32, P, I32, P, I64, P]),
    "oscar_bf16_decode_attn": (C.c_int, [SHAPE, P, I32, P, I32, P, I32, P, I64, P, P, SZ, P]),
    "oscar_hbm_copy": (C.c_int, [P, P, SZ, P]),
    "oscar_hbm_read": (C.c_int, [P, I64, P, I64, P, I32, P]),
    "oscar_hbm_read_nt": (C.c_int, [P, I64, P, I64, P, I32, P]),
    "oscar_gpu_wait": (C.c_int, [I64, P]),
    "oscar_event_create": (C.c_int, [C.POINTER(P)]),
    "oscar_event_destroy": (C.c_int, [P]),
    "oscar_event_elapsed_ms": (C.c_int, [P, P, C.POINTER(C.c_float)]),
    "oscar_quantize_append_timed": (C.c_int, [SHAPE, P, P, P, P, I64, P, P, I32, P, I32, P, P, I64, P, P, P, P, P]),
    "oscar_decode_attn_timed": (C.c_int, [SHAPE, P, P, P, I32, P, I32, P, I32, P, I64, P, P, P, P, SZ, P, P, P]),
    "oscar_decode_step": (C.c_int, [SHAPE, P, P, P, P, P, I32, P, I32, P, I32, P, I64, P, P, P, P, SZ, P]),
    "oscar_decode_step_timed": (C.c_int, [SHAPE, P, P, P, P, P, I32, P, I32, P, I32, P, I64, P, P, P, P, SZ, P, P,
                                          P]),
    "oscar_bf16_decode_attn_timed": (C.c_int, [SHAPE, P, I32, P, I32, P, I32, P, I64, P, P, SZ, P, P, P]),
    "oscar_strerror": (C.c_char_p, [C.c_int]),
}


def load(path: str = LIB_PATH) -> C.CDLL:
    # One process must hold exactly one HIP runtime.  torch ships its own
    # libamdhip64 (same SONAME as ROCm's); importing torch first makes the
    # library's libamdhip64.so.7 dependency bind to that already-loaded copy.
    # Loading the library first would pull in ROCm's copy and torch would then
    # load a second one.
    import torch  # noqa: F401

    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m kv_cache_int2_amd.build` "
            "(there is no CPU fallback)")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()
