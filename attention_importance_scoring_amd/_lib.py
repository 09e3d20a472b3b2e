"""ctypes loader for libspeckv.so and the C declarations of include/speckv.h.

Argument marshalling only: every step of the scoring path runs in the HIP
library.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

c_int32, c_int64, c_float, c_size_t, c_void_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

STATUS_NAMES = {
    0: "SKV_OK", 1: "SKV_ERR_NULL", 2: "SKV_ERR_SHAPE", 3: "SKV_ERR_DTYPE", 4: "SKV_ERR_PARAM",
    5: "SKV_ERR_WORKSPACE", 6: "SKV_ERR_ALIGN", 7: "SKV_ERR_ALIAS", 8: "SKV_ERR_HIP", 9: "SKV_ERR_INTERNAL",
}
SKV_F32, SKV_BF16 = 0, 1
SKV_POOL_NONE, SKV_POOL_MAX, SKV_POOL_AVG = 0, 1, 2
SKV_AGG_SUM, SKV_AGG_MAX = 0, 1

# Every symbol include/speckv.h declares.
EXPORTED = (
    "speckv_status_string", "speckv_workspace_bytes", "speckv_n_keep", "speckv_scores", "speckv_select",
    "speckv_compact", "specpc_gather_tokens", "speckv_scores_rows", "speckv_compact_rows", "specpc_token_scores",
    "speckv_decode_workspace_bytes", "speckv_decode_attention", "speckv_profile_enable", "speckv_profile_count",
    "speckv_profile_read", "speckv_scores_noalloc",
)


class Shape(ctypes.Structure):
    """Mirror of skv_shape."""
    _fields_ = [
        ("n_layers", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
        ("n_in", c_int64), ("kv_head_stride", c_int64), ("n_window", c_int32), ("n_lookahead", c_int32),
        ("scale", c_float), ("dtype", c_int32), ("aggregation", c_int32), ("per_query_head", c_int32),
    ]


_LIB = None


def load(path: str | None = None):
    """Load the HIP library (once) and declare its signatures."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library {p} is not built; run python -m attention_importance_scoring_amd.build")
    lib = ctypes.CDLL(p)
    S = ctypes.POINTER(Shape)
    lib.speckv_status_string.restype = ctypes.c_char_p
    lib.speckv_status_string.argtypes = [c_int32]
    lib.speckv_workspace_bytes.restype = c_int32
    lib.speckv_workspace_bytes.argtypes = [S, c_int32, ctypes.POINTER(c_size_t)]
    lib.speckv_n_keep.restype = c_int32
    lib.speckv_n_keep.argtypes = [S, c_int32, ctypes.POINTER(c_int64)]
    lib.speckv_scores.restype = c_int32
    lib.speckv_scores.argtypes = [S, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.speckv_scores_noalloc.restype = c_int32
    lib.speckv_scores_noalloc.argtypes = [S, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.speckv_select.restype = c_int32
    lib.speckv_select.argtypes = [S, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t,
                                  c_void_p]
    lib.speckv_compact.restype = c_int32
    lib.speckv_compact.argtypes = [S, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_size_t,
                                   c_void_p]
    lib.specpc_gather_tokens.restype = c_int32
    lib.specpc_gather_tokens.argtypes = [S, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p]
    lib.speckv_scores_rows.restype = c_int32
    lib.speckv_scores_rows.argtypes = [S, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.speckv_compact_rows.restype = c_int32
    lib.speckv_compact_rows.argtypes = [S, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p,
                                        c_void_p]
    lib.specpc_token_scores.restype = c_int32
    lib.specpc_token_scores.argtypes = [S, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                        c_void_p]
    lib.speckv_decode_workspace_bytes.restype = c_int32
    lib.speckv_decode_workspace_bytes.argtypes = [S, c_int64, ctypes.POINTER(c_size_t)]
    lib.speckv_decode_attention.restype = c_int32
    lib.speckv_decode_attention.argtypes = [S, c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                            c_void_p]
    lib.speckv_profile_enable.restype = c_int32
    lib.speckv_profile_enable.argtypes = [c_int32]
    lib.speckv_profile_count.restype = c_int32
    lib.speckv_profile_count.argtypes = []
    lib.speckv_profile_read.restype = c_int32
    lib.speckv_profile_read.argtypes = [c_int32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(c_int64),
                                        ctypes.POINTER(ctypes.c_double)]
    if path is None:
        _LIB = lib
    return lib
