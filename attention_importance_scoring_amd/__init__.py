"""MI355X (gfx950) SpecKV / SpecPC importance scoring, KV compaction and
decode attention over the compacted cache.

Thin Python binding over the C ABI in include/speckv.h (libspeckv.so): the
functions below carry the C names, turn torch device tensors into pointers
and a status code into an exception, and do nothing else.  PyTorch provides
device memory and streams only.  There is no CPU fallback: the HIP library
must be built and the tensors must live on the GPU.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import SKV_AGG_MAX, SKV_AGG_SUM, SKV_BF16, SKV_F32, SKV_POOL_AVG, SKV_POOL_MAX, SKV_POOL_NONE, Shape  # noqa: F401

__all__ = [
    "Shape", "SpecKVError", "make_shape", "speckv_workspace_bytes", "speckv_n_keep", "speckv_scores",
    "speckv_scores_noalloc",
    "speckv_select", "speckv_compact", "specpc_gather_tokens", "specpc_token_scores",
    "speckv_decode_workspace_bytes", "speckv_decode_attention", "profile_enable", "profile_read",
    "SKV_F32", "SKV_BF16", "SKV_POOL_NONE", "SKV_POOL_MAX", "SKV_POOL_AVG", "SKV_AGG_SUM", "SKV_AGG_MAX",
]


class SpecKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.load().speckv_status_string(status).decode()
        super().__init__(f"{where}: {_lib.STATUS_NAMES.get(status, status)} ({msg})")


def _check(status: int, where: str):
    if status != 0:
        raise SpecKVError(status, where)


def make_shape(n_layers, n_q_heads, n_kv_heads, head_dim, n_in, n_window, n_lookahead, dtype,
               kv_head_stride=0, scale=0.0, aggregation=0, per_query_head=0) -> Shape:
    return Shape(n_layers, n_q_heads, n_kv_heads, head_dim, n_in, kv_head_stride, n_window, n_lookahead, scale, dtype,
                 aggregation, per_query_head)


def _ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()


def speckv_workspace_bytes(shape: Shape, C_max: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.load().speckv_workspace_bytes(ctypes.byref(shape), C_max, ctypes.byref(out)), "speckv_workspace_bytes")
    return out.value


def speckv_n_keep(shape: Shape, C_max: int) -> int:
    out = ctypes.c_int64(0)
    _check(_lib.load().speckv_n_keep(ctypes.byref(shape), C_max, ctypes.byref(out)), "speckv_n_keep")
    return out.value


def speckv_scores(shape: Shape, q_obs, k, scores, workspace, stream=None):
    w, wb = _ws(workspace)
    _check(_lib.load().speckv_scores(ctypes.byref(shape), _ptr(q_obs, "q_obs"), _ptr(k, "k"), _ptr(scores, "scores"),
                                     w, wb, _stream(stream)), "speckv_scores")


def speckv_scores_noalloc(shape: Shape, q_obs, k, scores, stream=None):
    """speckv_scores with the library's fixed per-GPU scratch instead of a workspace."""
    _check(_lib.load().speckv_scores_noalloc(ctypes.byref(shape), _ptr(q_obs, "q_obs"), _ptr(k, "k"),
                                             _ptr(scores, "scores"), _stream(stream)), "speckv_scores_noalloc")


def speckv_select(shape: Shape, scores, C_max: int, pool: int, pool_kernel: int, kept, pooled, workspace,
                  stream=None):
    w, wb = _ws(workspace)
    _check(_lib.load().speckv_select(ctypes.byref(shape), _ptr(scores, "scores"), C_max, pool, pool_kernel,
                                     _ptr(kept, "kept"), _ptr(pooled, "pooled"), w, wb, _stream(stream)),
           "speckv_select")


def speckv_compact(shape: Shape, k, v, kept, n_keep: int, k_out, v_out, workspace, stream=None):
    w, wb = _ws(workspace)
    _check(_lib.load().speckv_compact(ctypes.byref(shape), _ptr(k, "k"), _ptr(v, "v"), _ptr(kept, "kept"), n_keep,
                                      _ptr(k_out, "k_out"), _ptr(v_out, "v_out"), w, wb, _stream(stream)),
           "speckv_compact")


def specpc_gather_tokens(shape: Shape, k, v, tokens, n_tokens: int, k_out, v_out, stream=None):
    _check(_lib.load().specpc_gather_tokens(ctypes.byref(shape), _ptr(k, "k"), _ptr(v, "v"), _ptr(tokens, "tokens"),
                                            n_tokens, _ptr(k_out, "k_out"), _ptr(v_out, "v_out"), _stream(stream)),
           "specpc_gather_tokens")


def speckv_scores_rows(shape: Shape, q_obs, k, rows, n_src_rows: int, scores, workspace, stream=None):
    w, wb = _ws(workspace)
    _check(_lib.load().speckv_scores_rows(ctypes.byref(shape), _ptr(q_obs, "q_obs"), _ptr(k, "k"), _ptr(rows, "rows"),
                                          n_src_rows, _ptr(scores, "scores"), w, wb, _stream(stream)),
           "speckv_scores_rows")


def speckv_compact_rows(shape: Shape, k, v, rows, n_src_rows: int, kept, n_keep: int, k_out, v_out, stream=None):
    _check(_lib.load().speckv_compact_rows(ctypes.byref(shape), _ptr(k, "k"), _ptr(v, "v"), _ptr(rows, "rows"),
                                           n_src_rows, _ptr(kept, "kept"), n_keep, _ptr(k_out, "k_out"),
                                           _ptr(v_out, "v_out"), _stream(stream)),
           "speckv_compact_rows")


def specpc_token_scores(shape: Shape, l_skip: int, q_win, k, query_weights, token_scores, workspace, stream=None):
    w, wb = _ws(workspace)
    _check(_lib.load().specpc_token_scores(ctypes.byref(shape), l_skip, _ptr(q_win, "q_win"), _ptr(k, "k"),
                                           _ptr(query_weights, "query_weights"), _ptr(token_scores, "token_scores"),
                                           w, wb, _stream(stream)), "specpc_token_scores")


def speckv_decode_workspace_bytes(shape: Shape, n_rows: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.load().speckv_decode_workspace_bytes(ctypes.byref(shape), n_rows, ctypes.byref(out)),
           "speckv_decode_workspace_bytes")
    return out.value


def speckv_decode_attention(shape: Shape, n_rows: int, q, k, v, out, workspace, stream=None):
    w, wb = _ws(workspace)
    _check(_lib.load().speckv_decode_attention(ctypes.byref(shape), n_rows, _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"),
                                               _ptr(out, "out"), w, wb, _stream(stream)), "speckv_decode_attention")


def profile_enable(on: bool):
    _check(_lib.load().speckv_profile_enable(1 if on else 0), "speckv_profile_enable")


def profile_read() -> dict:
    """{kernel name: (launches, total event ms)} for the launches recorded so far."""
    lib = _lib.load()
    out = {}
    for i in range(lib.speckv_profile_count()):
        name, n, ms = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_double()
        _check(lib.speckv_profile_read(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)), "speckv_profile_read")
        out[name.value.decode()] = (n.value, ms.value)
    return out
