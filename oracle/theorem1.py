"""Theorem-1 form of the score-error bound (paper notes "Draft-based
Approximate Inference for LLMs", section "Key designs", SpecKV paragraph:
the importance-score error is proportional to the draft embedding error,
||s - s_hat||_2 <= eps * ||W_q W_k^T||_2).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Reading: s are the pre-softmax scores of one query embedding x against the
input keys, s = (x W_q)(X W_k)^T with the scale absorbed; the draft replaces
x by x_hat with ||x - x_hat||_2 <= eps.  Then
||s - s_hat||_2 <= eps * ||W_q W_k^T||_2 * ||X||_2, and the printed form is
the case ||X||_2 <= 1.
"""
from __future__ import annotations

import numpy as np

from .speckv import row_logits


def pre_softmax_scores(q, k, scale: float = 1.0) -> np.ndarray:
    """s_j = scale * <q, k_j> for one query q [d] against keys k [n, d]: the
    logits the SpecKV scoring itself feeds to its softmax (row_logits)."""
    return row_logits(np.asarray(q, dtype=np.float64)[None, :], k, scale)[0]


def theorem1_bound(eps: float, w_q, w_k, x_keys=None) -> float:
    """eps * ||W_q W_k^T||_2 (times ||X||_2 when the key embeddings are given)."""
    m = np.asarray(w_q, dtype=np.float64) @ np.asarray(w_k, dtype=np.float64).T
    b = eps * np.linalg.norm(m, 2)
    if x_keys is not None:
        b *= np.linalg.norm(np.asarray(x_keys, dtype=np.float64), 2)
    return float(b)
