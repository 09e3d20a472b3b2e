"""fp64 oracle for decode attention over a (compacted) KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: paper notes "Draft-based Approximate Inference for LLMs", section
"Background": attention cost grows with the context and the KV cache with
its length, which is what dropping KV pairs saves; section "Key designs",
SpecKV paragraph: after the prefill the target keeps only the top C_max
pairs plus the window and generates over that cache.  Generation step:
each query head's new query attends over the cached rows of its KV head.

Readings taken here (the pages do not print the attention formula):
* standard scaled dot-product attention, softmax over every cached row
  (no mask: all cached rows precede the new token), scale 1/sqrt(d);
* query head hq reads KV head hq // G (G = Hq / Hkv), or its own cache when
  the cache holds one set of rows per query head;
* the new token's own K/V, when the caller wants it attended, is one more
  cached row (appended by the caller).
"""
from __future__ import annotations

import numpy as np

from .speckv import default_scale


def head_attention(q_rows, k_rows, v_rows, scale: float) -> np.ndarray:
    """q_rows [n_q, d], k_rows [n, d], v_rows [n, d_v] -> out [n_q, d_v]:
    out_i = sum_j softmax_j(scale * <q_i, k_j>) v_j."""
    q = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    v = np.asarray(v_rows, dtype=np.float64)
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v


def decode_attention(q, k, v, n_rows: int | None = None, scale: float | None = None) -> np.ndarray:
    """q [L, Hq, d] (one new query per query head); k, v [L, H, n, d] with
    H = Hkv (shared by groups of G = Hq / H query heads) or H = Hq.  Only
    the first n_rows cached rows are attended (default: all).
    Returns float64 [L, Hq, d]."""
    L, Hq, d = q.shape
    Lk, H, n, dk = k.shape
    assert L == Lk and d == dk and Hq % H == 0 and v.shape[:3] == k.shape[:3]
    n_rows = n if n_rows is None else int(n_rows)
    assert 1 <= n_rows <= n
    G = Hq // H
    tau = default_scale(d) if scale is None else float(scale)
    out = np.empty((L, Hq, v.shape[3]), dtype=np.float64)
    for layer in range(L):
        for hq in range(Hq):
            h = hq // G
            out[layer, hq] = head_attention(q[layer, hq][None], k[layer, h, :n_rows], v[layer, h, :n_rows], tau)[0]
    return out


def error_scale(q, k, v, n_rows: int | None = None, scale: float | None = None) -> np.ndarray:
    """sum_j P_j |v_j| per (layer, query head, component): the size of the
    terms an output component is the sum of (the natural unit for its
    rounding error).  Same shapes and reading as decode_attention."""
    return decode_attention(q, k, np.abs(np.asarray(v, dtype=np.float64)), n_rows, scale)
