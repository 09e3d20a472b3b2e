"""Theorem-1 check (paper notes "Draft-based Approximate Inference for LLMs",
section "Key designs", SpecKV: ||s - s_hat||_2 <= eps ||W_q W_k^T||_2 on the
pre-softmax scores when the query embedding is perturbed by at most eps).

The scores are the logits of the oracle's own SpecKV scoring (row_logits,
the input of its softmax); key embeddings X have orthonormal rows, so
||X||_2 = 1 and the printed form applies.
"""
import numpy as np
import pytest

import oracle


def _setup(seed, d_model=64, d=16, n=12):
    rng = np.random.default_rng(seed)
    w_q = rng.standard_normal((d_model, d)) / np.sqrt(d_model)
    w_k = rng.standard_normal((d_model, d)) / np.sqrt(d_model)
    m = w_q @ w_k.T
    u, _, vt = np.linalg.svd(m)
    # X: orthonormal rows whose span contains the top right singular vector of W_q W_k^T
    basis = np.concatenate([vt[:1], rng.standard_normal((n - 1, d_model))], axis=0)
    qmat, _ = np.linalg.qr(basis.T)
    X = qmat.T[:n]
    x = rng.standard_normal(d_model)
    return rng, w_q, w_k, u, X, x


@pytest.mark.parametrize("seed", range(5))
def test_bound_holds_for_random_perturbations(seed):
    rng, w_q, w_k, _, X, x = _setup(seed)
    assert np.linalg.norm(X, 2) == pytest.approx(1.0, abs=1e-12)
    K = X @ w_k
    s = oracle.pre_softmax_scores(x @ w_q, K)
    for eps in (1e-3, 0.1, 2.0):
        for _ in range(20):
            e = rng.standard_normal(x.shape)
            e *= eps / np.linalg.norm(e)
            s_hat = oracle.pre_softmax_scores((x + e) @ w_q, K)
            assert np.linalg.norm(s - s_hat) <= oracle.theorem1_bound(eps, w_q, w_k) * (1 + 1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_bound_is_attained_along_top_singular_direction(seed):
    _, w_q, w_k, u, X, x = _setup(seed)
    K = X @ w_k
    eps = 0.37
    e = eps * u[:, 0]
    gap = np.linalg.norm(oracle.pre_softmax_scores(x @ w_q, K) - oracle.pre_softmax_scores((x + e) @ w_q, K))
    assert gap == pytest.approx(oracle.theorem1_bound(eps, w_q, w_k), rel=1e-10)


def test_scale_enters_linearly():
    _, w_q, w_k, _, X, x = _setup(0)
    s1 = oracle.pre_softmax_scores(x @ w_q, X @ w_k, 1.0)
    s2 = oracle.pre_softmax_scores(x @ w_q, X @ w_k, 0.125)
    np.testing.assert_allclose(s2, 0.125 * s1, rtol=1e-15)


def test_bound_holds_on_the_logits_the_scoring_softmax_uses():
    # the same perturbation seen through row_probabilities: its log-probabilities
    # are the logits up to a per-row constant, so the centred log-probabilities
    # move by at most the bound too (centring is an orthogonal projection)
    import scipy.special
    rng, w_q, w_k, _, X, x = _setup(7)
    K = X @ w_k
    p = oracle.row_probabilities((x @ w_q)[None], K, 1.0)[0]
    np.testing.assert_allclose(p, scipy.special.softmax(oracle.pre_softmax_scores(x @ w_q, K)), rtol=1e-13)
    for eps in (1e-3, 0.1, 1.0):
        e = rng.standard_normal(x.shape)
        e *= eps / np.linalg.norm(e)
        p_hat = oracle.row_probabilities(((x + e) @ w_q)[None], K, 1.0)[0]
        d = np.log(p) - np.log(p_hat)
        assert np.linalg.norm(d - d.mean()) <= oracle.theorem1_bound(eps, w_q, w_k) * (1 + 1e-10)
