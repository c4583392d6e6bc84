"""ctypes loader for libba_att.so (the C ABI declared in include/ba_att.h).

Loading fails loudly: there is no fallback implementation of any entry point.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libba_att.so")

# (name, restype, argtypes) for every symbol of the C ABI
_i32, _f32, _f64, _sz, _p = ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = [
    ("ba_att_num_blocks", _i32, [_i32, _i32]),
    ("ba_att_keep_count", _i32, [_i32, _f64]),
    ("ba_att_select_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32]),
    ("ba_att_select", ctypes.c_int,
     [_i32, _i32, _i32, _i32, _i32, _f32, _f64, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    ("ba_att_select_noalloc", ctypes.c_int,
     [_i32, _i32, _i32, _i32, _i32, _f32, _f64, _p, _p, _p, _p, _p, _p, _p]),
    ("ba_att_mask_to_index", ctypes.c_int, [_i32, _i32, _i32, _p, _i32, _p, _p, _p]),
    ("ba_att_forward", ctypes.c_int,
     [_i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p, _i32, _p, _i32, _p, _p]),
    ("ba_att_forward_queued", ctypes.c_int,
     [_i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p, _i32, _p, _i32, _p, _p, _p]),
    ("ba_att_forward_split_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32]),
    ("ba_att_forward_split_parts", _i32, [_i32, _i32, _i32, _i32, _i32]),
    ("ba_att_forward_split", ctypes.c_int,
     [_i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p, _i32, _i32, _p, _i32, _p, _p, _sz, _p]),
    ("ba_att_merge", ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _p, _p, _p, _i32, _p, _p]),
    ("ba_att_forward_ext", ctypes.c_int,
     [_i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p, _i32, _p, _p, _p, _i32, _p, _p]),
    ("ba_att_dense", ctypes.c_int, [_i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p, _i32, _p, _p]),
    ("ba_att_block_map", ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p, _p]),
    ("ba_att_score_full_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32]),
    ("ba_att_score_full", ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p, _sz, _p]),
    ("ba_att_rank_agreement", ctypes.c_int, [_i32, _i32, _i32, _i32, _p, _p, _p, _p, _p]),
    ("ba_att_status_string", ctypes.c_char_p, [ctypes.c_int]),
]

_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Loads the built library once; raises if it is missing or incomplete."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"BA-Att HIP library not found at {path}; build it with "
            "`python -m block_sparse_attention_ba_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)  # AttributeError if a symbol is missing
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ---- libba_peaks.so: machine-peak microbenchmarks (include/ba_peaks.h), for
# the rooflines' context only
PEAKS_PATH = os.path.join(_PKG, "libba_peaks.so")
PEAK_SIGNATURES = [
    ("ba_peak_read", ctypes.c_int, [_p, _sz, _p, _i32, _i32, _p]),
    ("ba_peak_copy", ctypes.c_int, [_p, _p, _sz, _i32, _p]),
    ("ba_peak_mfma_bf16", ctypes.c_int, [_p, _i32, _i32, _f32, _p]),
    ("ba_peak_mfma_bf16_random", ctypes.c_int, [_p, _i32, _i32, ctypes.c_uint32, _p]),
]

_peaks = None


def load_peaks(path: str | None = None) -> ctypes.CDLL:
    """Loads the built microbenchmark library once; raises if it is missing."""
    global _peaks
    if _peaks is not None:
        return _peaks
    path = path or PEAKS_PATH
    if not os.path.exists(path):
        raise ImportError(f"peak microbenchmark library not found at {path}; build it with "
                          "`python -m block_sparse_attention_ba_amd.build`")
    lib = ctypes.CDLL(path)
    for name, res, args in PEAK_SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _peaks = lib
    return lib
