"""Pins for the SpecKV scoring oracle (oracle/speckv.py).

Each test fixes a fact that follows from the definition in the paper notes
"Draft-based Approximate Inference for LLMs" (section "Key designs", SpecKV)
by a route other than the oracle's own code: hand-derived closed forms,
scipy's softmax, the logistic function, invariants, and an independent
pure-Python fsum implementation on tiny inputs.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_example_exact_fractions():
    # d = 4 so the default scale is 1/2.  Row q1 sees logits (ln 3, 0, 0) and row q2
    # sees (0, ln 2, 0); by hand the softmax rows are (3/5, 1/5, 1/5) and (1/4, 1/2, 1/4),
    # so the column sums are (17/20, 7/10, 9/20).  Key 3 is the window key: it is not in
    # the normaliser, so its huge logit must change nothing.
    d = 4
    k = np.zeros((1, 1, 4, d))
    k[0, 0, 0, 0] = 2 * math.log(3)
    k[0, 0, 1, 1] = 2 * math.log(2)
    k[0, 0, 3] = [100.0, 100.0, 0.0, 0.0]
    q = np.zeros((1, 1, 2, d))
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 1, 1] = 1.0
    got = oracle.speckv_scores(q, k, n_window=1)
    want = [Fraction(3, 5) + Fraction(1, 4), Fraction(1, 5) + Fraction(1, 2), Fraction(1, 5) + Fraction(1, 4)]
    np.testing.assert_allclose(got[0, 0], [float(x) for x in want], rtol=0, atol=1e-15)


def test_hand_example_gqa_group_sums_heads():
    # Two query heads share the KV head; the second head swaps the two rows, so each
    # column sum doubles: (17/10, 7/5, 9/10).
    d = 4
    k = np.zeros((1, 1, 3, d))
    k[0, 0, 0, 0] = 2 * math.log(3)
    k[0, 0, 1, 1] = 2 * math.log(2)
    q = np.zeros((1, 2, 2, d))
    q[0, 0, 0, 0] = q[0, 1, 1, 0] = 1.0
    q[0, 0, 1, 1] = q[0, 1, 0, 1] = 1.0
    got = oracle.speckv_scores(q, k, n_window=0)
    np.testing.assert_allclose(got[0, 0], [1.7, 1.4, 0.9], rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", range(3))
def test_rows_sum_to_one_and_columns_total_group_times_nobs(seed):
    rng_shape = (2, 6, 5, 16)  # L, Hq, n_obs, d
    q = _rand(rng_shape, seed)
    k = _rand((2, 2, 40, 16), seed + 100) * 2.0
    P = oracle.row_probabilities(q[0, 0], k[0, 0, :33], oracle.default_scale(16))
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    s = oracle.speckv_scores(q, k, n_window=7)
    assert s.shape == (2, 2, 33)
    G, n_obs = 3, 5
    np.testing.assert_allclose(s.sum(axis=-1), G * n_obs, rtol=1e-13)
    assert (s >= 0).all()


def test_single_row_equals_scipy_softmax():
    q = _rand((1, 1, 1, 32), 1)
    k = _rand((1, 1, 50, 32), 2) * 3
    tau = 1 / math.sqrt(32)
    got = oracle.speckv_scores(q, k, n_window=4)[0, 0]
    want = scipy.special.softmax(tau * (k[0, 0, :46] @ q[0, 0, 0]))
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-300)


def test_equal_keys_give_uniform_scores():
    q = _rand((1, 4, 6, 8), 3)
    k = np.tile(_rand((8,), 4), (1, 2, 30, 1))
    s = oracle.speckv_scores(q, k, n_window=5)
    np.testing.assert_allclose(s, 2 * 6 / 25, rtol=1e-13)


def test_two_keys_is_logistic_of_logit_gap():
    q = _rand((1, 3, 4, 16), 5)
    k = _rand((1, 1, 3, 16), 6) * 2
    tau = 0.25
    s = oracle.speckv_scores(q, k, n_window=1, scale=tau)[0, 0]
    rows = q[0].reshape(-1, 16)
    gap = tau * rows @ (k[0, 0, 0] - k[0, 0, 1])
    np.testing.assert_allclose(s[0], scipy.special.expit(gap).sum(), rtol=1e-13)
    np.testing.assert_allclose(s[1], scipy.special.expit(-gap).sum(), rtol=1e-13)


def test_gqa_mapping_contiguous_groups():
    # query head hq belongs to KV head hq // G: check against explicit one-head slices
    q = _rand((1, 6, 3, 8), 7)
    k = _rand((1, 3, 20, 8), 8)
    s = oracle.speckv_scores(q, k, n_window=2)
    for h in range(3):
        want = sum(oracle.speckv_scores(q[:, [2 * h + g]], k[:, [h]], n_window=2)[0, 0] for g in range(2))
        np.testing.assert_allclose(s[0, h], want, rtol=1e-13)
    # and a different head's keys would give a different answer
    assert not np.allclose(s[0, 0], s[0, 1])


def test_window_keys_not_in_normaliser_but_last_prefix_key_is():
    q = _rand((1, 2, 4, 8), 9)
    k = _rand((1, 1, 20, 8), 10)
    base = oracle.speckv_scores(q, k, n_window=5)
    k2 = k.copy()
    k2[0, 0, 15:] *= 50.0
    np.testing.assert_array_equal(oracle.speckv_scores(q, k2, n_window=5), base)
    k3 = k.copy()
    k3[0, 0, 14] += 5.0
    assert not np.allclose(oracle.speckv_scores(q, k3, n_window=5), base)


def test_lookahead_rows_count():
    # every observation row (window and lookahead alike) adds one unit of mass
    q = _rand((1, 1, 9, 8), 11)
    k = _rand((1, 1, 30, 8), 12)
    full = oracle.speckv_scores(q, k, n_window=3)
    part = oracle.speckv_scores(q[:, :, :3], k, n_window=3)
    assert abs(full.sum() - 9) < 1e-12 and abs(part.sum() - 3) < 1e-12
    assert (full >= part - 1e-15).all()


def test_key_permutation_equivariance():
    q = _rand((1, 2, 3, 8), 13)
    k = _rand((1, 1, 25, 8), 14)
    perm = np.random.default_rng(0).permutation(20)
    kp = k.copy()
    kp[0, 0, :20] = k[0, 0, perm]
    np.testing.assert_allclose(oracle.speckv_scores(q, kp, 5)[0, 0], oracle.speckv_scores(q, k, 5)[0, 0][perm],
                               rtol=1e-13)


def _fsum_scores(q, k, n_window, tau):
    """Independent brute force with math.fsum and explicit loops."""
    L, Hq, n_obs, d = q.shape
    _, Hkv, n_in, _ = k.shape
    G = Hq // Hkv
    n_pre = n_in - n_window
    out = [[[0.0] * n_pre for _ in range(Hkv)] for _ in range(L)]
    for l in range(L):
        for hq in range(Hq):
            h = hq // G
            for i in range(n_obs):
                logits = [tau * math.fsum(q[l, hq, i, t] * k[l, h, j, t] for t in range(d)) for j in range(n_pre)]
                m = max(logits)
                z = math.fsum(math.exp(x - m) for x in logits)
                for j in range(n_pre):
                    out[l][h][j] += math.exp(logits[j] - m) / z
    return np.array(out)


@pytest.mark.parametrize("seed", range(4))
def test_bruteforce_fsum_tiny(seed):
    rng = np.random.default_rng(seed)
    L, Hkv, G = 2, 2, 2
    n_obs, d, n_in, n_window = 3, 4, 11, 3
    q = rng.standard_normal((L, Hkv * G, n_obs, d)) * 2
    k = rng.standard_normal((L, Hkv, n_in, d)) * 2
    np.testing.assert_allclose(oracle.speckv_scores(q, k, n_window),
                               _fsum_scores(q, k, n_window, 0.5), rtol=1e-12)


def test_planted_heavy_hitters_recovered_tiny_config():
    from attention_importance_scoring_amd import workloads as w
    cfg = w.TINY_FP32_2K
    inp = w.speckv_inputs(cfg, seed=1)
    q = w.to_numpy_f64(inp["q_obs"])
    k = w.to_numpy_f64(inp["k"])
    s = oracle.speckv_scores(q, k, cfg.n_window)
    kept, _ = oracle.speckv_select(s, cfg.C_max, cfg.n_window, "max", cfg.pool_kernel)
    # planted keys are the rows that are far from N(0, I): norm >> sqrt(d)
    norms = np.linalg.norm(k[0, 0, :cfg.n_pre], axis=-1)
    planted = np.nonzero(norms > 2.5 * math.sqrt(cfg.head_dim))[0]
    assert len(planted) == 9 and planted[0] == 0
    assert set(planted.tolist()) <= set(kept[0, 0].tolist())


# ---- variants: max over the observation rows, one kept set per query head ----

def test_max_aggregation_hand_example():
    # Same rows as the hand example: softmax rows (3/5, 1/5, 1/5) and (1/4, 1/2, 1/4),
    # so the column maxima are (3/5, 1/2, 1/4).
    d = 4
    k = np.zeros((1, 1, 4, d))
    k[0, 0, 0, 0] = 2 * math.log(3)
    k[0, 0, 1, 1] = 2 * math.log(2)
    k[0, 0, 3] = [100.0, 100.0, 0.0, 0.0]
    q = np.zeros((1, 1, 2, d))
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 1, 1] = 1.0
    got = oracle.speckv_scores(q, k, n_window=1, aggregation="max")
    np.testing.assert_allclose(got[0, 0], [0.6, 0.5, 0.25], rtol=0, atol=1e-15)


def test_max_aggregation_equal_keys_is_uniform_probability():
    # every row is uniform over the n_pre keys, so every column maximum is 1 / n_pre
    q = _rand((1, 3, 4, 8), 5)
    k = np.tile(_rand((1, 1, 1, 8), 6), (1, 1, 50, 1))
    got = oracle.speckv_scores(q, k, n_window=10, aggregation="max")
    np.testing.assert_allclose(got, 1.0 / 40, rtol=1e-13)


def test_max_aggregation_single_row_equals_sum():
    q = _rand((2, 1, 1, 16), 7)
    k = _rand((2, 1, 30, 16), 8)
    np.testing.assert_allclose(oracle.speckv_scores(q, k, 4, aggregation="max"), oracle.speckv_scores(q, k, 4),
                               rtol=1e-14)


def test_per_query_head_scores_add_up_to_kv_head_scores():
    # the KV-head sum runs over the group's query heads, so it is the sum of the per-head scores
    q = _rand((2, 6, 5, 16), 9)
    k = _rand((2, 2, 40, 16), 10) * 2
    per_head = oracle.speckv_scores(q, k, 7, per_query_head=True)
    grouped = oracle.speckv_scores(q, k, 7)
    assert per_head.shape == (2, 6, 33)
    np.testing.assert_allclose(per_head.reshape(2, 2, 3, 33).sum(axis=2), grouped, rtol=1e-13)
    np.testing.assert_allclose(per_head.sum(-1), 5.0, rtol=1e-13)  # n_obs rows per query head


@pytest.mark.parametrize("seed", range(3))
def test_bruteforce_max_and_per_query_head_tiny(seed):
    rng = np.random.default_rng(seed)
    L, Hkv, G, n_obs, d, n_in, n_window = 2, 2, 3, 3, 4, 10, 2
    q = rng.standard_normal((L, Hkv * G, n_obs, d)) * 2
    k = rng.standard_normal((L, Hkv, n_in, d)) * 2
    n_pre = n_in - n_window
    want_max = np.zeros((L, Hkv, n_pre))
    want_pqh = np.zeros((L, Hkv * G, n_pre))
    for l in range(L):
        for hq in range(Hkv * G):
            h = hq // G
            for i in range(n_obs):
                logits = [0.5 * math.fsum(q[l, hq, i, t] * k[l, h, j, t] for t in range(d)) for j in range(n_pre)]
                m = max(logits)
                z = math.fsum(math.exp(x - m) for x in logits)
                for j in range(n_pre):
                    p = math.exp(logits[j] - m) / z
                    want_max[l, h, j] = max(want_max[l, h, j], p)
                    want_pqh[l, hq, j] += p
    np.testing.assert_allclose(oracle.speckv_scores(q, k, n_window, aggregation="max"), want_max, rtol=1e-12)
    np.testing.assert_allclose(oracle.speckv_scores(q, k, n_window, per_query_head=True), want_pqh, rtol=1e-12)


def test_planted_heavy_hitters_recovered_qwen32b_shape_64k():
    # The 64K Qwen2.5-32B-shaped workload (rank-8 keys plus 1 % planted heavy
    # hitters and the sink), two layers in fp64: every kept prefix key lies
    # within the pooling half-width of a planted key.  The 656 planted keys
    # per head make about 4600 plateau slots against C_max = 256, so only the
    # strongest fit: the kept keys form 256 / 7 (about 37) whole plateaus.
    import numpy as np
    from attention_importance_scoring_amd import workloads as w
    cfg = w.QWEN32B_64K
    inp = w.speckv_inputs(cfg, seed=3, layers=[0, 63])
    s = oracle.speckv_scores(w.to_numpy_f64(inp["q_obs"]), w.to_numpy_f64(inp["k"]), cfg.n_window)
    kept, _ = oracle.speckv_select(s, cfg.C_max, cfg.n_window, "max", cfg.pool_kernel)
    r = cfg.pool_kernel // 2
    for i in range(2):
        for h in range(cfg.n_kv_heads):
            planted = inp["planted"][i][h].numpy()
            assert len(planted) == cfg.n_in // 100 + 1 and planted[0] == 0
            prefix = kept[i, h, :cfg.C_max]
            dist = np.abs(prefix[:, None] - planted[None, :]).min(axis=1)
            assert (dist <= r).all(), f"layer {i} head {h}: kept keys far from every planted key"
            near = np.abs(planted[:, None] - prefix[None, :]).min(axis=1) == 0
            assert near.sum() >= cfg.C_max // cfg.pool_kernel, "too few planted keys kept"
