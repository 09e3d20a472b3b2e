"""Pins for the SpecKV-PC cascade oracle (oracle/cascade.py).

Source: paper notes "Draft-based Approximate Inference for LLMs", section
"Key designs", SpecKV-PC paragraph (SpecPC cuts the prompt first, SpecKV then
cuts the target's cache over the shorter prompt).  The two stages are pinned
on their own in test_oracle_specpc.py and test_oracle_speckv.py; these tests
pin how they are joined: which index space each stage works in, which tokens
form the SpecKV window, and which rows end up in the final cache.
"""
import numpy as np

import oracle
from oracle.cascade import gather_tokens, speckv_pc_cascade


def _rand(shape, seed, s=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * s


def test_gather_tokens_is_take_along_the_token_axis():
    kv = _rand((2, 3, 17, 5), 1)
    tokens = np.array([16, 0, 3, 3, 9])
    np.testing.assert_array_equal(gather_tokens(kv, tokens), np.take(kv, tokens, axis=2))


def test_hand_example_positions():
    # Draft: one layer, one head, W = 1 (the last position sees every key), query e0,
    # keys c_j * e0: token scores are softmax(c / 2).  With no pooling and k_top = 5
    # SpecPC keeps the five largest c_j: positions 1, 4, 6, 9, 11.
    n_in, d = 12, 4
    c = np.array([0.0, 5.0, 1.0, 0.5, 6.0, 0.0, 7.0, 2.0, 0.0, 4.5, 1.5, 8.0])
    q_win = np.zeros((1, 1, 1, d))
    q_win[0, 0, 0, 0] = 1.0
    k_draft = np.zeros((1, 1, n_in, d))
    k_draft[0, 0, :, 0] = c
    # Target: one layer, one head, n_window 2, C_max 1.  On the compressed prompt the
    # window is tokens 9 and 11, the prefix is tokens 1, 4, 6; the target key of token 4
    # has the largest logit, so the final cache holds positions 4, 9, 11.
    t = np.zeros(n_in)
    t[[1, 4, 6]] = [1.0, 3.0, 2.0]
    t[[10, 11]] = [50.0, 50.0]  # large, but window keys are never scored
    q_obs = np.zeros((1, 1, 3, d))
    q_obs[0, 0, :, 1] = 1.0
    k_t = np.zeros((1, 1, n_in, d))
    k_t[0, 0, :, 1] = t
    v_t = _rand((1, 1, n_in, d), 2)
    out = speckv_pc_cascade(q_win, k_draft, 0, 5, q_obs, k_t, v_t, n_window=2, C_max=1, pool_mode="none",
                            pool_kernel=1)
    np.testing.assert_array_equal(out["tokens"], [1, 4, 6, 9, 11])
    np.testing.assert_array_equal(out["kept"][0, 0], [1, 3, 4])
    np.testing.assert_array_equal(out["positions"][0, 0], [4, 9, 11])
    np.testing.assert_array_equal(out["v"][0, 0], v_t[0, 0, [4, 9, 11]])
    # SpecKV scores cover the three prefix tokens and sum to the number of observation rows
    np.testing.assert_allclose(out["scores"][0, 0].sum(), 3.0, rtol=1e-14)
    assert out["scores"][0, 0].argmax() == 1


def test_full_budget_is_plain_speckv():
    # k_top >= n_in: SpecPC keeps every token, so the cascade is SpecKV on the full prompt.
    Ld, L, n_in, d = 3, 2, 40, 8
    q_win = _rand((Ld, 4, 6, d), 3)
    k_draft = _rand((Ld, 2, n_in, d), 4)
    q_obs = _rand((L, 4, 5, d), 5)
    k_t = _rand((L, 2, n_in, d), 6, 1.5)
    v_t = _rand((L, 2, n_in, d), 7)
    out = speckv_pc_cascade(q_win, k_draft, 1, n_in + 3, q_obs, k_t, v_t, n_window=4, C_max=9)
    np.testing.assert_array_equal(out["tokens"], np.arange(n_in))
    scores = oracle.speckv_scores(q_obs, k_t, 4)
    kept, _ = oracle.speckv_select(scores, 9, 4)
    kc, vc = oracle.speckv_compact(k_t, v_t, kept)
    np.testing.assert_array_equal(out["scores"], scores)
    np.testing.assert_array_equal(out["kept"], kept)
    np.testing.assert_array_equal(out["positions"], kept)
    np.testing.assert_array_equal(out["k"], kc)
    np.testing.assert_array_equal(out["v"], vc)


def test_invariants_random():
    Ld, L, n_in, d, n_window, k_top, C_max = 4, 3, 300, 16, 8, 64, 12
    q_win = _rand((Ld, 6, 16, d), 8)
    k_draft = _rand((Ld, 2, n_in, d), 9, 2.0)
    q_obs = _rand((L, 8, 10, d), 10)
    k_t = _rand((L, 4, n_in, d), 11, 2.0)
    v_t = _rand((L, 4, n_in, d), 12)
    out = speckv_pc_cascade(q_win, k_draft, 1, k_top, q_obs, k_t, v_t, n_window, C_max)
    tokens = out["tokens"]
    assert len(tokens) == k_top and (np.diff(tokens) > 0).all()
    pos = out["positions"]
    assert pos.shape == (L, 4, C_max + n_window)
    for layer in range(L):
        for h in range(4):
            p = pos[layer, h]
            assert (np.diff(p) > 0).all()
            assert np.isin(p, tokens).all()
            np.testing.assert_array_equal(p[-n_window:], tokens[-n_window:])
            np.testing.assert_array_equal(out["k"][layer, h], k_t[layer, h][p])
            np.testing.assert_array_equal(out["v"][layer, h], v_t[layer, h][p])
    np.testing.assert_allclose(out["scores"].sum(-1), 2 * 10, rtol=1e-12)  # G * n_obs per KV head
