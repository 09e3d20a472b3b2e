"""fp64 oracle for the SpecKV-PC cascade: SpecPC compresses the prompt, then
SpecKV drops KV pairs of the target's cache over the compressed prompt.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: paper notes "Draft-based Approximate Inference for LLMs", section
"Key designs", SpecKV-PC paragraph: the prompt is first cut to a token budget
by SpecPC (2048 tokens in the example) and the target's KV cache over that
shorter prompt is then cut further by SpecKV (256 pairs in the example); the
target only ever processes the compressed prompt.

Readings taken here (the pages do not fix them):
* the compressed prompt is the SpecPC kept tokens in their original order;
* the target's K/V over the compressed prompt are given as the rows of a
  target cache over the full prompt at the kept token positions (the target's
  prefill of the compressed prompt is a model forward, outside the scoring
  path; a real prefill would also renumber positions, which synthetic keys
  without rotary embedding do not see);
* the SpecKV window is the last n_window tokens of the compressed prompt,
  and SpecKV's observation queries are the target's queries of that window
  plus its lookahead tokens, given as input.
"""
from __future__ import annotations

import numpy as np

from .speckv import speckv_compact, speckv_scores, speckv_select
from .specpc import specpc_select, specpc_token_scores


def gather_tokens(kv, tokens) -> np.ndarray:
    """kv: [L, H, n_in, d]; tokens: [n_tok] positions.  out[l, h, t] = kv[l, h, tokens[t]]
    for every layer and head (one token list shared by all of them), exact copy."""
    kv = np.asarray(kv)
    L, H = kv.shape[:2]
    out = np.empty((L, H, len(tokens)) + kv.shape[3:], dtype=kv.dtype)
    for layer in range(L):
        for h in range(H):
            for t, j in enumerate(tokens):
                out[layer, h, t] = kv[layer, h, j]
    return out


def speckv_pc_cascade(q_win, k_draft, l_skip: int, k_top: int, q_obs, k_target, v_target, n_window: int,
                      C_max: int, pool_mode: str = "max", pool_kernel: int = 7, weights=None, scale=None):
    """SpecPC on the draft stack, then SpecKV on the target cache of the kept tokens.

    q_win [Ld, Hq_d, W, d_d], k_draft [Ld, Hkv_d, n_in, d_d]: the draft's window
    queries and keys over the full prompt.  q_obs [L, Hq, n_obs, d]: the
    target's observation queries; k_target, v_target [L, Hkv, n_in, d]: the
    target cache over the full prompt (rows taken at the kept tokens).

    Returns a dict: tokens [n_tok] (SpecPC kept positions, ascending),
    scores [L, Hkv, n_tok - n_window] (SpecKV scores on the compressed
    prompt), kept [L, Hkv, n_keep] (indices into the compressed prompt),
    positions = tokens[kept] (original prompt positions), k, v [L, Hkv,
    n_keep, d] (the final cache).
    """
    ts = specpc_token_scores(q_win, k_draft, l_skip, weights, scale)
    tokens, _ = specpc_select(ts, k_top, pool_mode, pool_kernel)
    k_c = gather_tokens(k_target, tokens)
    v_c = gather_tokens(v_target, tokens)
    scores = speckv_scores(q_obs, k_c, n_window, scale)
    kept, _ = speckv_select(scores, C_max, n_window, pool_mode, pool_kernel)
    kc, vc = speckv_compact(k_c, v_c, kept)
    return {"token_scores": ts, "tokens": tokens, "scores": scores, "kept": kept, "positions": tokens[kept],
            "k": kc, "v": vc}
