"""Pins for the SpecPC oracle (oracle/specpc.py).

Source: paper notes "Draft-based Approximate Inference for LLMs", section
"Key designs", SpecPC paragraph (window of queries with weights falling away
from the end, skipped shallow layers, mean then max).
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle


def _rand(shape, seed, s=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * s


def test_hand_example():
    # one layer, one head, n_in = 2, W = 2, d = 4 (scale 1/2).  Row 0 sits at position 0
    # and sees only key 0: (1, 0).  Row 1 sees logits (ln 3, 0): (3/4, 1/4).
    # Default weights are (0.1, 1): scores = (max(0.1, 0.75), max(0, 0.25)) = (0.75, 0.25).
    q = np.zeros((1, 1, 2, 4))
    q[0, 0, 1, 0] = 1.0
    q[0, 0, 0] = [5.0, -3.0, 2.0, 0.0]
    k = np.zeros((1, 1, 2, 4))
    k[0, 0, 0, 0] = 2 * math.log(3)
    k[0, 0, 1] = [0.0, 7.0, 0.0, 0.0]  # only visible to row 1, and orthogonal to its query
    np.testing.assert_allclose(oracle.specpc_token_scores(q, k, 0), [0.75, 0.25], rtol=0, atol=1e-15)


def test_rows_are_causal_distributions():
    q = _rand((2, 4, 6, 8), 1)
    k = _rand((2, 2, 20, 8), 2, 2.0)
    P = oracle.causal_window_probabilities(q[0, 0], k[0, 0], 0.3)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
    for i in range(6):
        assert (P[i, 20 - 6 + i + 1:] == 0).all()
    abar = oracle.specpc_attention_mean(q, k, 1)
    np.testing.assert_allclose(abar.sum(axis=1), 1.0, atol=1e-14)


def test_single_row_single_head_is_scipy_softmax():
    q = _rand((1, 1, 1, 16), 3)
    k = _rand((1, 1, 30, 16), 4, 2.0)
    got = oracle.specpc_token_scores(q, k, 0)
    np.testing.assert_allclose(got, scipy.special.softmax(0.25 * k[0, 0] @ q[0, 0, 0]), rtol=1e-13)


def test_last_token_only_seen_by_last_row():
    q = _rand((3, 2, 5, 8), 5)
    k = _rand((3, 1, 12, 8), 6)
    abar = oracle.specpc_attention_mean(q, k, 1)
    s = oracle.specpc_token_scores(q, k, 1)
    assert s[-1] == pytest.approx(1.0 * abar[-1, -1], rel=1e-15)


def test_layers_below_l_skip_are_ignored():
    q = _rand((4, 2, 5, 8), 7)
    k = _rand((4, 1, 15, 8), 8)
    base = oracle.specpc_token_scores(q, k, 2)
    q2, k2 = q.copy(), k.copy()
    q2[:2] = _rand((2, 2, 5, 8), 9, 5.0)
    k2[:2, :, 3] = 40.0  # a loud heavy hitter in a skipped layer
    np.testing.assert_array_equal(oracle.specpc_token_scores(q2, k2, 2), base)
    k3 = k.copy()
    k3[2, :, 3] += 3.0
    assert not np.allclose(oracle.specpc_token_scores(q, k3, 2), base)


def test_unit_weights_give_plain_max_and_weights_scale_rows():
    q = _rand((2, 2, 4, 8), 10)
    k = _rand((2, 1, 10, 8), 11)
    abar = oracle.specpc_attention_mean(q, k, 0)
    np.testing.assert_allclose(oracle.specpc_token_scores(q, k, 0, weights=np.ones(4)), abar.max(axis=0), rtol=1e-15)
    w = oracle.default_query_weights(4)
    np.testing.assert_allclose(w, [0.1, 0.4, 0.7, 1.0])
    assert oracle.default_query_weights(1).tolist() == [1.0]


def test_mean_over_duplicated_heads_is_unchanged():
    q = _rand((2, 2, 4, 8), 12)
    k = _rand((2, 1, 10, 8), 13)
    base = oracle.specpc_token_scores(q, k, 0)
    q2 = np.concatenate([q, q], axis=1)  # same heads twice, same KV head
    np.testing.assert_allclose(oracle.specpc_token_scores(q2, k, 0), base, rtol=1e-14)


def _fsum_specpc(q, k, l_skip, w, tau):
    L, Hq, W, d = q.shape
    _, Hkv, n_in, _ = k.shape
    G = Hq // Hkv
    acc = [[0.0] * n_in for _ in range(W)]
    for l in range(l_skip, L):
        for hq in range(Hq):
            for i in range(W):
                pos = n_in - W + i
                logits = [tau * math.fsum(q[l, hq, i, t] * k[l, hq // G, j, t] for t in range(d)) for j in range(pos + 1)]
                m = max(logits)
                z = math.fsum(math.exp(x - m) for x in logits)
                for j in range(pos + 1):
                    acc[i][j] += math.exp(logits[j] - m) / z
    n_maps = (L - l_skip) * Hq
    return np.array([max(w[i] * acc[i][j] / n_maps for i in range(W)) for j in range(n_in)])


@pytest.mark.parametrize("seed", range(3))
def test_bruteforce_fsum_tiny(seed):
    q = _rand((3, 4, 3, 4), seed, 1.5)
    k = _rand((3, 2, 7, 4), seed + 50, 1.5)
    w = oracle.default_query_weights(3)
    np.testing.assert_allclose(oracle.specpc_token_scores(q, k, 1), _fsum_specpc(q, k, 1, w, 0.5), rtol=1e-12)


def test_specpc_select_no_forced_window():
    s = np.linspace(1.0, 0.0, 40)
    kept, _ = oracle.specpc_select(s, 5, "max", 1)
    assert kept.tolist() == [0, 1, 2, 3, 4]


# ---- n_lookahead > 1: draft rows at the end of the window, draft keys in their normaliser ----

def test_lookahead_hand_example():
    # n_in = 2 input tokens, n_lookahead = 2: one draft token at position 2; W = 2 rows at
    # positions 1 and 2, d = 4, scale 1/2.  Row 0 (position 1, input) sees keys 0, 1 with
    # logits (0, ln 3): (1/4, 3/4).  Row 1 (position 2, draft) sees keys 0, 1, 2 with logits
    # (ln 2, 0, ln 5): (2/8, 1/8, 5/8); the input columns keep (1/4, 1/8).
    # Weights (0.1, 1): scores = (max(0.025, 0.25), max(0.075, 0.125)) = (0.25, 0.125).
    q = np.zeros((1, 1, 2, 4))
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 1, 1] = 1.0
    k = np.zeros((1, 1, 3, 4))
    k[0, 0, 1, 0] = 2 * math.log(3)
    k[0, 0, 0, 1] = 2 * math.log(2)
    k[0, 0, 2, 1] = 2 * math.log(5)
    abar = oracle.specpc_attention_mean(q, k, 0, n_in=2)
    np.testing.assert_allclose(abar, [[0.25, 0.75], [0.25, 0.125]], rtol=1e-14)
    np.testing.assert_allclose(oracle.specpc_token_scores(q, k, 0, n_in=2), [0.25, 0.125], rtol=1e-14)


def test_lookahead_row_sums_and_reduction():
    L, Hq, Hkv, W, d, n_in, n_la = 3, 4, 2, 6, 8, 30, 4
    q = _rand((L, Hq, W, d), 31)
    k = _rand((L, Hkv, n_in + n_la - 1, d), 32, 2.0)
    abar = oracle.specpc_attention_mean(q, k, 1, n_in=n_in)
    sums = abar.sum(axis=1)
    # input rows (the first W - (n_la - 1)) see only input keys: they sum to one
    np.testing.assert_allclose(sums[:W - (n_la - 1)], 1.0, atol=1e-14)
    # draft rows lose exactly the mass their (causal) draft keys take
    full = oracle.specpc_attention_mean(q, k, 1, n_in=n_in + n_la - 1)
    np.testing.assert_allclose(sums + full[:, n_in:].sum(axis=1), 1.0, atol=1e-14)
    assert (sums[W - (n_la - 1):] < 1.0).all()
    # n_in = all keys is the n_lookahead = 1 form
    np.testing.assert_array_equal(oracle.specpc_token_scores(q, k, 1, n_in=n_in + n_la - 1),
                                  oracle.specpc_token_scores(q, k, 1))


def test_lookahead_bruteforce_fsum():
    W, d, n_in, n_la = 3, 3, 5, 3
    q = _rand((1, 1, W, d), 33)
    k = _rand((1, 1, n_in + n_la - 1, d), 34)
    tau = 1 / math.sqrt(d)
    n_keys = n_in + n_la - 1
    w = oracle.default_query_weights(W)
    want = [0.0] * n_in
    for i in range(W):
        pos = n_keys - W + i
        logits = [tau * math.fsum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d)) for j in range(pos + 1)]
        z = math.fsum(math.exp(x) for x in logits)
        for j in range(n_in):
            if j <= pos:
                want[j] = max(want[j], w[i] * math.exp(logits[j]) / z)
    got = oracle.specpc_token_scores(q, k, 0, n_in=n_in)
    np.testing.assert_allclose(got, want, rtol=1e-13)
