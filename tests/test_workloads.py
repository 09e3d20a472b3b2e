"""Seeded input generators: determinism, shapes, planted structure."""
import math

import numpy as np
import torch

import oracle
from attention_importance_scoring_amd import workloads as w


def test_same_seed_same_bytes_and_shapes():
    cfg = w.reduced(w.LLAMA8B_16K, n_layers=2, n_in=512, C_max=64)
    a = w.speckv_inputs(cfg, seed=2)
    b = w.speckv_inputs(cfg, seed=2)
    c = w.speckv_inputs(cfg, seed=3)
    for key in ("q_obs", "k", "v"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])
    assert a["q_obs"].shape == (2, 32, 96, 128) and a["q_obs"].dtype == torch.bfloat16
    assert a["k"].shape == (2, 8, 512, 128)


def test_padded_head_stride_views():
    cfg = w.reduced(w.TINY_FP32_2K, n_in=300)
    a = w.speckv_inputs(cfg, seed=1)
    b = w.speckv_inputs(cfg, seed=1, kv_head_stride=300 * 64 + 40)
    assert torch.equal(a["k"], b["k"]) and b["k_buf"].shape[-1] == 300 * 64 + 40


def test_one_percent_heavy_hitters_are_recovered_llama_layer():
    # One layer of the Llama-3.1-8B-shaped 16K workload: every kept prefix key lies
    # within the pooling half-width of a planted key (or the sink).
    cfg = w.LLAMA8B_16K
    inp = w.speckv_inputs(cfg, seed=2, layers=[0])
    q = w.to_numpy_f64(inp["q_obs"])
    k = w.to_numpy_f64(inp["k"])
    s = oracle.speckv_scores(q, k, cfg.n_window)
    kept, _ = oracle.speckv_select(s, cfg.C_max, cfg.n_window, "max", cfg.pool_kernel)
    for h in range(cfg.n_kv_heads):
        norms = np.linalg.norm(k[0, h, :cfg.n_pre], axis=-1)
        planted = np.nonzero(norms > 2.0 * math.sqrt(cfg.head_dim))[0]
        assert len(planted) == cfg.n_in // 100 + 1
        prefix_kept = kept[0, h, :cfg.C_max]
        dist = np.abs(prefix_kept[:, None] - planted[None, :]).min(axis=1)
        assert (dist <= cfg.pool_kernel // 2).all()


def test_specpc_inputs_shapes():
    cfg = w.SPECPC_DRAFT_32K
    small = w.dataclasses.replace(cfg, n_layers=5, n_in=1024, window=64)
    inp = w.specpc_inputs(small, seed=5)
    assert inp["q_win"].shape == (5, 14, 64, 64) and inp["k"].shape == (5, 2, 1024, 64)
