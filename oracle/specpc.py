"""fp64 oracle for SpecPC token scoring over a draft attention stack.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: paper notes "Draft-based Approximate Inference for LLMs", section
"Key designs", SpecPC paragraph: the draft's attention activations
A (layers x heads x (n_in + n_lookahead - 1) x n_in) estimate token
importance; a large window of queries is used with weights that fall with
distance from the end; the first l_skip layers are skipped; aggregation is a
mean first, then a max.  Section "Loss / training strategy": local pooling
keeps tokens contiguous.

Readings taken here (the pages do not fix them):
* the query axis of A has n_in + n_lookahead - 1 positions: the input
  tokens, then the draft's generated tokens but the last (which is never
  fed back); the window is the last W positions of that axis.  With
  n_lookahead = 1 (the pages' chosen setting) all window rows are input
  queries; with n_lookahead > 1 the last n_lookahead - 1 window rows are
  draft tokens;
* the keys are those of the same positions; a window row's causal softmax
  runs over every key up to its own position, draft keys included, and A
  (hence the token scores) keeps only the n_in input-token columns;
* each row is the draft's causal softmax over keys j <= its position
  (scale 1/sqrt(d));
* the mean runs over the used layers (l >= l_skip) and all query heads;
* the weights multiply the averaged rows before the max over rows; the
  default weights rise linearly from 0.1 at the far edge of the window to
  1 at its end;
* no tokens are force-kept; the top k tokens by (pooled score desc, index
  asc) are kept, in ascending order.
"""
from __future__ import annotations

import numpy as np

from .speckv import default_scale, pool1d, select_kept


def default_query_weights(W: int) -> np.ndarray:
    """w_i = 0.1 + 0.9 * i / (W - 1): 1 at the last window row, 0.1 at the first."""
    if W == 1:
        return np.ones(1)
    return 0.1 + 0.9 * np.arange(W, dtype=np.float64) / (W - 1)


def causal_window_probabilities(q_win_head, k_head, scale: float) -> np.ndarray:
    """Causal attention rows of the W window queries of one draft head.

    q_win_head: [W, d]; k_head: [n_keys, d], the keys of every position of
    the query axis (n_keys = n_in + n_lookahead - 1); row i sits at position
    n_keys - W + i.  Returns P [W, n_keys]: P[i, j] = softmax over
    j <= pos_i of scale*<q_i, k_j>, and 0 for j > pos_i.
    """
    q = np.asarray(q_win_head, dtype=np.float64)
    k = np.asarray(k_head, dtype=np.float64)
    W, n_keys = q.shape[0], k.shape[0]
    pos = n_keys - W + np.arange(W)
    s = scale * (q @ k.T)
    future = np.arange(n_keys)[None, :] > pos[:, None]
    s[future] = -np.inf
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def specpc_attention_mean(q_win, k, l_skip: int, scale: float | None = None, n_in: int | None = None) -> np.ndarray:
    """Mean of the causal window attention over layers l >= l_skip and all
    query heads, on the input-token columns.  q_win: [L, Hq, W, d];
    k: [L, Hkv, n_keys, d] (input keys, then n_lookahead - 1 draft keys);
    n_in: input tokens (default n_keys, i.e. n_lookahead = 1).
    Returns [W, n_in]."""
    L, Hq, W, d = q_win.shape
    Lk, Hkv, n_keys, _ = k.shape
    n_in = n_keys if n_in is None else int(n_in)
    assert L == Lk and Hq % Hkv == 0 and 0 <= l_skip < L and W <= n_keys and 1 <= n_in <= n_keys
    G = Hq // Hkv
    tau = default_scale(d) if scale is None else float(scale)
    acc = np.zeros((W, n_in), dtype=np.float64)
    for layer in range(l_skip, L):
        for hq in range(Hq):
            acc += causal_window_probabilities(q_win[layer, hq], k[layer, hq // G], tau)[:, :n_in]
    return acc / ((L - l_skip) * Hq)


def specpc_token_scores(q_win, k, l_skip: int, weights=None, scale: float | None = None,
                        n_in: int | None = None) -> np.ndarray:
    """score[j] = max_i w_i * Abar[i, j] over the window rows.  Returns [n_in]
    (n_in: input tokens, default all keys; see specpc_attention_mean)."""
    abar = specpc_attention_mean(q_win, k, l_skip, scale, n_in)
    W = abar.shape[0]
    w = default_query_weights(W) if weights is None else np.asarray(weights, dtype=np.float64)
    return (w[:, None] * abar).max(axis=0)


def specpc_select(token_scores, k_top: int, pool_mode: str = "max", pool_kernel: int = 7):
    """Pool the token scores, keep the k_top best tokens (no forced window),
    ascending.  Returns (kept tokens int64, pooled float64)."""
    pooled = pool1d(np.asarray(token_scores, dtype=np.float64), pool_kernel, pool_mode)
    return select_kept(pooled, k_top, 0), pooled
