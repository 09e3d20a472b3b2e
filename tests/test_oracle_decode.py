"""Pins for the decode-attention oracle (oracle/decode.py).

Source: paper notes "Draft-based Approximate Inference for LLMs", sections
"Background" and "Key designs" (SpecKV: generation runs over the kept KV
pairs).  Each pin is fixed by the mathematics of softmax attention, not by
re-running the oracle's own formula: closed forms, scipy's softmax on a
single head, brute force with math.fsum, and the GQA head mapping.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle.decode import decode_attention, error_scale


def _rand(shape, seed, s=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * s


def test_single_row_returns_its_value():
    q, k, v = _rand((2, 4, 8), 1), _rand((2, 2, 1, 8), 2), _rand((2, 2, 1, 8), 3)
    out = decode_attention(q, k, v)
    for hq in range(4):
        np.testing.assert_array_equal(out[:, hq], v[:, hq // 2, 0])


def test_equal_keys_give_the_mean_value():
    q = _rand((1, 3, 16), 4)
    k = np.tile(_rand((1, 1, 1, 16), 5), (1, 3, 9, 1))
    v = _rand((1, 3, 9, 16), 6)
    np.testing.assert_allclose(decode_attention(q, k, v), v.mean(axis=2), rtol=1e-13, atol=1e-15)


def test_single_head_matches_scipy_softmax():
    q, k, v = _rand((1, 1, 32), 7), _rand((1, 1, 50, 32), 8, 2.0), _rand((1, 1, 50, 32), 9)
    w = scipy.special.softmax(k[0, 0] @ q[0, 0] / math.sqrt(32))
    np.testing.assert_allclose(decode_attention(q, k, v)[0, 0], w @ v[0, 0], rtol=1e-12, atol=1e-14)


def test_bruteforce_fsum_with_scale_and_prefix_rows():
    q, k, v = _rand((1, 2, 3), 10), _rand((1, 1, 6, 3), 11), _rand((1, 1, 6, 3), 12)
    n_rows, tau = 4, 0.7
    got = decode_attention(q, k, v, n_rows=n_rows, scale=tau)
    for hq in range(2):
        logits = [tau * math.fsum(q[0, hq, c] * k[0, 0, j, c] for c in range(3)) for j in range(n_rows)]
        e = [math.exp(x) for x in logits]
        z = math.fsum(e)
        for c in range(3):
            want = math.fsum(e[j] * v[0, 0, j, c] for j in range(n_rows)) / z
            assert got[0, hq, c] == pytest.approx(want, rel=1e-13, abs=1e-15)


def test_gqa_mapping_reads_the_group_kv_head():
    # constant V per KV head: every query head of group h returns head h's constant
    L, Hq, H, n, d = 2, 6, 3, 7, 4
    q, k = _rand((L, Hq, d), 13), _rand((L, H, n, d), 14)
    v = np.zeros((L, H, n, d))
    for layer in range(L):
        for h in range(H):
            v[layer, h] = 10 * layer + h
    out = decode_attention(q, k, v)
    for hq in range(Hq):
        np.testing.assert_allclose(out[:, hq], (10 * np.arange(L) + hq // 2)[:, None] * np.ones(d), rtol=1e-14)


def test_dominant_key_and_convexity():
    q = np.zeros((1, 1, 4))
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, 5, 4))
    k[0, 0, 3, 0] = 200.0  # logit 100 above the rest: weight 1 - 4e-44
    v = _rand((1, 1, 5, 4), 15)
    np.testing.assert_allclose(decode_attention(q, k, v)[0, 0], v[0, 0, 3], rtol=1e-15, atol=1e-15)
    # any output lies inside the componentwise range of the attended values
    q2, k2, v2 = _rand((1, 4, 8), 16), _rand((1, 1, 30, 8), 17, 3.0), _rand((1, 1, 30, 8), 18)
    out = decode_attention(q2, k2, v2)
    assert (out <= v2[0, 0].max(axis=0) + 1e-15).all() and (out >= v2[0, 0].min(axis=0) - 1e-15).all()


def test_error_scale_bounds_the_output():
    q, k, v = _rand((2, 4, 8), 19), _rand((2, 2, 12, 8), 20), _rand((2, 2, 12, 8), 21)
    out, es = decode_attention(q, k, v), error_scale(q, k, v)
    assert (np.abs(out) <= es + 1e-15).all()
    # with non-negative values the two coincide
    np.testing.assert_allclose(error_scale(q, k, np.abs(v)), decode_attention(q, k, np.abs(v)), rtol=1e-15)


def test_compacted_cache_equals_full_cache_restricted_to_kept_rows():
    # decode over the compacted cache = attention over the kept rows of the full cache
    L, Hq, H, n, d = 1, 4, 2, 40, 8
    q, k, v = _rand((L, Hq, d), 22), _rand((L, H, n, d), 23), _rand((L, H, n, d), 24)
    kept = np.stack([[np.sort(np.random.default_rng(25 + h).choice(n, 9, replace=False)) for h in range(H)]])
    kc, vc = oracle.speckv_compact(k, v, kept)
    got = decode_attention(q, kc, vc)
    for hq in range(Hq):
        rows = kept[0, hq // 2]
        w = scipy.special.softmax(k[0, hq // 2, rows] @ q[0, hq] / math.sqrt(d))
        np.testing.assert_allclose(got[0, hq], w @ v[0, hq // 2, rows], rtol=1e-12, atol=1e-14)
