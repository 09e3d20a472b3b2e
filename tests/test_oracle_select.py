"""Pins for pooling, top-C_max selection and compaction in the oracle.

Source: paper notes "Draft-based Approximate Inference for LLMs", section
"Key designs" (SpecKV keeps the top C_max pairs plus the window pairs) and
section "Loss / training strategy" (local pooling).
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.ndimage

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("kernel", [1, 3, 5, 7, 9])
@pytest.mark.parametrize("n", [1, 2, 5, 64, 301])
def test_max_pool_equals_scipy_maximum_filter(kernel, n):
    x = np.random.default_rng(n * 13 + kernel).standard_normal((3, n))
    got = oracle.pool1d(x, kernel, "max")
    want = scipy.ndimage.maximum_filter1d(x, size=kernel, axis=-1, mode="nearest")
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("kernel", [1, 3, 7])
@pytest.mark.parametrize("n", [1, 4, 50])
def test_avg_pool_truncated_window_bruteforce(kernel, n):
    x = np.random.default_rng(n + kernel).standard_normal(n)
    r = kernel // 2
    want = [np.mean(x[max(0, j - r):min(n, j + r + 1)]) for j in range(n)]
    np.testing.assert_allclose(oracle.pool1d(x, kernel, "avg"), want, rtol=1e-14)


def _beats(vals, b, a):
    return vals[b] > vals[a] or (vals[b] == vals[a] and b < a)


def _rank_rule(vals, C_max):
    """A key is kept iff fewer than C_max keys beat it (O(n^2) counting)."""
    n = len(vals)
    return [a for a in range(n) if sum(_beats(vals, b, a) for b in range(n) if b != a) < C_max]


def _subset_rule(vals, C_max):
    """Max-sum subset of size C_max; among equal sums, lexicographically smallest."""
    best, best_key = None, None
    for sub in itertools.combinations(range(len(vals)), C_max):
        key = (-sum(vals[i] for i in sub), sub)
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return list(best)


@pytest.mark.parametrize("seed", range(8))
def test_select_bruteforce_subsets_with_ties(seed):
    rng = np.random.default_rng(seed)
    n_pre = int(rng.integers(1, 11))
    vals = rng.integers(0, 4, n_pre).astype(np.float64)  # small integers: many exact ties
    for C_max in range(0, n_pre + 2):
        n_window = int(rng.integers(0, 3))
        kept = oracle.select_kept(vals, C_max, n_window)
        c = min(C_max, n_pre)
        want_top = _subset_rule(vals.tolist(), c) if c > 0 else []
        assert kept.tolist() == sorted(want_top) + list(range(n_pre, n_pre + n_window))


def test_select_rank_rule_larger():
    rng = np.random.default_rng(5)
    vals = rng.integers(0, 50, 600).astype(np.float64)
    for C_max in (1, 17, 256, 599, 600):
        assert oracle.select_kept(vals, C_max, 0).tolist() == _rank_rule(vals.tolist(), C_max)


def test_select_uniform_scores_keep_lowest_indices():
    kept = oracle.select_kept(np.full(100, 0.25), 7, 4)
    assert kept.tolist() == list(range(7)) + list(range(100, 104))


def test_select_invariants_and_edge_cases():
    rng = np.random.default_rng(3)
    vals = rng.random(500)
    kept = oracle.select_kept(vals, 64, 16)
    assert len(kept) == oracle.n_keep(516, 16, 64) == 80
    assert (np.diff(kept) > 0).all()
    assert set(range(500, 516)) <= set(kept.tolist())
    assert oracle.select_kept(vals, 0, 3).tolist() == [500, 501, 502]
    assert oracle.select_kept(vals, 10_000, 2).tolist() == list(range(502))
    # the kept prefix keys are exactly the 64 largest
    assert set(kept[:64].tolist()) == set(np.argsort(-vals)[:64].tolist())


def test_pool_then_select_plateau_tie_break():
    # one spike at 10 becomes a 7-wide plateau 7..13 after max-pool(7); with C_max = 3
    # the three lowest plateau indices are kept.
    s = np.zeros((1, 1, 30))
    s[0, 0, 10] = 1.0
    kept, pooled = oracle.speckv_select(s, 3, 2, "max", 7)
    np.testing.assert_array_equal(pooled[0, 0, 7:14], 1.0)
    assert kept[0, 0].tolist() == [7, 8, 9, 30, 31]


def test_compact_rows_encode_their_index():
    L, H, n_in, d = 2, 3, 40, 4
    k = np.zeros((L, H, n_in, d), dtype=np.float32)
    k[..., 0] = np.arange(n_in)
    k[..., 1] = np.arange(H)[None, :, None]
    k[..., 2] = np.arange(L)[:, None, None]
    v = -k
    rng = np.random.default_rng(0)
    kept = np.stack([np.stack([np.sort(rng.choice(n_in, 9, replace=False)) for _ in range(H)]) for _ in range(L)])
    kc, vc = oracle.speckv_compact(k, v, kept)
    assert kc.dtype == np.float32
    np.testing.assert_array_equal(kc[..., 0], kept)
    np.testing.assert_array_equal(vc[..., 0], -kept)
    np.testing.assert_array_equal(kc[..., 1], np.broadcast_to(np.arange(H)[None, :, None], kept.shape))
    np.testing.assert_array_equal(kc[..., 2], np.broadcast_to(np.arange(L)[:, None, None], kept.shape))


def test_compact_per_query_head_reads_its_kv_head():
    # kept sets per query head: 6 query heads over 2 KV heads, head hq reads KV head hq // 3
    L, Hkv, G, n_in, d = 2, 2, 3, 30, 4
    k = np.zeros((L, Hkv, n_in, d), dtype=np.float32)
    k[..., 0] = np.arange(n_in)
    k[..., 1] = np.arange(Hkv)[None, :, None]
    v = k + 0.5
    rng = np.random.default_rng(1)
    kept = np.stack([np.stack([np.sort(rng.choice(n_in, 5, replace=False)) for _ in range(Hkv * G)])
                     for _ in range(L)])
    kc, vc = oracle.speckv_compact(k, v, kept)
    assert kc.shape == (L, Hkv * G, 5, d)
    np.testing.assert_array_equal(kc[..., 0], kept)
    np.testing.assert_array_equal(kc[..., 1], np.broadcast_to((np.arange(Hkv * G) // G)[None, :, None], kept.shape))
    np.testing.assert_array_equal(vc - kc, 0.5)


def test_kv_cache_size_closed_form_from_the_pages():
    with open(os.path.join(GOLDEN, "kv_cache_size_llama8b_128k.json")) as f:
        g = json.load(f)
    n_bytes = 2 * g["n_layers"] * g["n_kv_heads"] * g["head_dim"] * g["tokens"] * g["bytes_per_element"]
    assert n_bytes == 16 * 2**30
    assert n_bytes / 1e9 >= g["stated_lower_bound_gb"]
