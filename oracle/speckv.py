"""fp64 oracle for SpecKV: observation-query scoring, pooling, top-C_max
selection with window retention, and KV compaction.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: paper notes "Draft-based Approximate Inference for LLMs", section
"Key designs", SpecKV paragraph: the draft proposes n_lookahead tokens; the
target prefills input plus lookahead; for each head, the importance of every
KV pair is estimated from the cross-attention of the queries of the last
n_window input tokens and of the lookahead tokens against the remaining
input keys; the top C_max KV pairs are kept together with the window's pairs.
Section "Loss / training strategy": local pooling keeps selected tokens
contiguous.

All arithmetic is float64 on exactly converted inputs (bf16 and fp32 values
are exact in float64).
"""
from __future__ import annotations

import math

import numpy as np

_ROW_CHUNK = 64  # rows of the score matrix held at once (memory only; no reordering of the math)


def default_scale(head_dim: int) -> float:
    """Reading: the score scale is the usual 1/sqrt(d) of scaled dot-product
    attention (the pages do not print it)."""
    return 1.0 / math.sqrt(head_dim)


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def row_logits(q_rows, k_prefix, scale: float) -> np.ndarray:
    """Pre-softmax scores s_rj = scale * <q_r, k_j> of the observation rows
    q_rows [R, d] against the keys k_prefix [n, d]; returns [R, n].

    Reading: the usual scaled dot product, the scale applied after the
    product (the pages do not print the score formula)."""
    return scale * (_as_f64(q_rows) @ _as_f64(k_prefix).T)


def row_probabilities(q_rows, k_prefix, scale: float) -> np.ndarray:
    """Softmax of each observation query row over the remaining input keys.

    q_rows: [R, d]; k_prefix: [n_pre, d]. Returns P [R, n_pre] with
    P[r, j] = exp(s_rj - lse_r), s_rj = row_logits (scale * <q_r, k_j>),
    lse_r = m_r + log(sum_j exp(s_rj - m_r)), m_r = max_j s_rj.

    Reading: the normaliser of each row is the set of remaining input keys
    only (the keys that are scored), so every row sums to one over them.
    """
    s = row_logits(q_rows, k_prefix, scale)
    m = s.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
    return np.exp(s - lse)


def head_scores(q_group, k_prefix, scale: float, aggregation: str = "sum") -> np.ndarray:
    """Importance of each remaining input key for one KV head.

    q_group: [G, n_obs, d], the observation queries of the G query heads that
    share this KV head (window rows then lookahead rows, the order does not
    matter); k_prefix: [n_pre, d].

    aggregation "sum": score[j] = sum over query heads g and observation rows
    i of P_(g,i)[j].
    aggregation "max": score[j] = max over the same rows of P_(g,i)[j].

    Reading: the pages say the importance comes from the cross-attention of
    the observation queries; the default aggregation over queries and over
    the GQA group is a plain sum (a mean would rank identically).  The "max"
    variant takes the largest probability any observation row gives the key,
    the reduction the pages' SpecPC paragraph applies across its query rows.
    """
    if aggregation not in ("sum", "max"):
        raise ValueError(aggregation)
    q = _as_f64(q_group)
    rows = q.reshape(-1, q.shape[-1])
    k = _as_f64(k_prefix)
    score = np.zeros(k.shape[0], dtype=np.float64)
    for r0 in range(0, rows.shape[0], _ROW_CHUNK):
        p = row_probabilities(rows[r0:r0 + _ROW_CHUNK], k, scale)
        if aggregation == "sum":
            score += p.sum(axis=0)
        else:
            score = np.maximum(score, p.max(axis=0))
    return score


def speckv_scores(q_obs, k, n_window: int, scale: float | None = None, aggregation: str = "sum",
                  per_query_head: bool = False) -> np.ndarray:
    """Scores for every layer and KV head (or query head).

    q_obs: [L, Hq, n_obs, d]; k: [L, Hkv, n_in, d] (only the first
    n_pre = n_in - n_window rows of each head are scored).
    Query head hq belongs to KV head hq // G with G = Hq / Hkv.
    Returns float64 [L, Hkv, n_pre], or [L, Hq, n_pre] with per_query_head,
    where query head hq is scored alone against its KV head's keys.

    Reading (per_query_head): the pages estimate importance per attention
    head; the default keeps one set per KV head, shared by its query heads,
    and this variant keeps one per query head.
    """
    L, Hq, _, d = q_obs.shape
    Lk, Hkv, n_in, dk = k.shape
    assert L == Lk and d == dk and Hq % Hkv == 0 and 0 <= n_window <= n_in
    G = Hq // Hkv
    n_pre = n_in - n_window
    tau = default_scale(d) if scale is None else float(scale)
    if per_query_head:
        out = np.empty((L, Hq, n_pre), dtype=np.float64)
        for layer in range(L):
            for hq in range(Hq):
                out[layer, hq] = head_scores(q_obs[layer, hq:hq + 1], k[layer, hq // G, :n_pre], tau, aggregation)
        return out
    out = np.empty((L, Hkv, n_pre), dtype=np.float64)
    for layer in range(L):
        for h in range(Hkv):
            out[layer, h] = head_scores(q_obs[layer, h * G:(h + 1) * G], k[layer, h, :n_pre], tau, aggregation)
    return out


def pool1d(x, kernel: int, mode: str = "max") -> np.ndarray:
    """Local 1-D pooling along the last axis, stride 1, same length.

    out[j] = max (or mean) of x[j'] over |j' - j| <= kernel // 2 and
    0 <= j' < n.  Reading: windows are truncated at both ends (equivalent to
    -inf padding for max; the mean divides by the in-range count).
    mode "none" returns the input unchanged.
    """
    x = _as_f64(x)
    if mode == "none" or kernel == 1:
        return x.copy()
    assert kernel >= 1 and kernel % 2 == 1
    r = kernel // 2
    n = x.shape[-1]
    if mode == "max":
        out = x.copy()
        for off in range(1, r + 1):
            if off >= n:
                break
            out[..., :-off] = np.maximum(out[..., :-off], x[..., off:])
            out[..., off:] = np.maximum(out[..., off:], x[..., :-off])
        return out
    if mode == "avg":
        total = x.copy()
        count = np.ones(n, dtype=np.float64)
        for off in range(1, r + 1):
            if off >= n:
                break
            total[..., :-off] += x[..., off:]
            count[:-off] += 1
            total[..., off:] += x[..., :-off]
            count[off:] += 1
        return total / count
    raise ValueError(f"unknown pooling mode {mode!r}")


def n_keep(n_in: int, n_window: int, C_max: int) -> int:
    """Number of kept KV pairs per head: min(C_max, n_pre) + n_window."""
    return min(C_max, n_in - n_window) + n_window


def select_kept(pooled, C_max: int, n_window: int) -> np.ndarray:
    """Kept indices of one head, ascending.

    pooled: [n_pre] pooled importance of the remaining input keys.  Keeps the
    C_max best keys plus every window key n_pre .. n_pre + n_window - 1.

    Reading: "best" orders by pooled score descending and, among equal
    scores, by lower index first (pooling makes plateaus of equal values, so
    a deterministic tie rule is needed; the pages give none).  When
    C_max >= n_pre every prefix key is kept.
    """
    p = _as_f64(pooled)
    n_pre = p.shape[0]
    n_top = min(C_max, n_pre)
    order = np.argsort(-p, kind="stable")  # stable: equal scores keep index order
    top = np.sort(order[:n_top])
    window = np.arange(n_pre, n_pre + n_window)
    return np.concatenate([top, window]).astype(np.int64)


def speckv_select(scores, C_max: int, n_window: int, pool_mode: str = "max", pool_kernel: int = 7):
    """Pool then select for every head. scores: [L, Hkv, n_pre].
    Returns (kept [L, Hkv, n_keep] int64, pooled [L, Hkv, n_pre] float64)."""
    s = _as_f64(scores)
    pooled = pool1d(s, pool_kernel, pool_mode)
    L, Hkv, n_pre = s.shape
    kept = np.empty((L, Hkv, min(C_max, n_pre) + n_window), dtype=np.int64)
    for layer in range(L):
        for h in range(Hkv):
            kept[layer, h] = select_kept(pooled[layer, h], C_max, n_window)
    return kept, pooled


def compact_rows(rows, kept) -> np.ndarray:
    """Compacted cache of one head: out[t] = rows[kept[t]] (exact copy)."""
    rows = np.asarray(rows)
    out = np.empty((len(kept),) + rows.shape[1:], dtype=rows.dtype)
    for t, j in enumerate(kept):
        out[t] = rows[j]
    return out


def speckv_compact(k, v, kept):
    """k, v: [L, Hkv, n_in, d]; kept: [L, H, n_keep] with H = Hkv (one kept
    set per KV head) or H = Hq, a multiple of Hkv (one per query head, taken
    from KV head hq // (Hq / Hkv)).
    Returns (k_c, v_c) of shape [L, H, n_keep, d], same dtype as the input."""
    L, H = kept.shape[:2]
    Hkv = k.shape[1]
    assert H % Hkv == 0
    rep = H // Hkv
    kc = np.empty((L, H, kept.shape[2]) + k.shape[3:], dtype=k.dtype)
    vc = np.empty((L, H, kept.shape[2]) + v.shape[3:], dtype=v.dtype)
    for layer in range(L):
        for h in range(H):
            kc[layer, h] = compact_rows(k[layer, h // rep], kept[layer, h])
            vc[layer, h] = compact_rows(v[layer, h // rep], kept[layer, h])
    return kc, vc
