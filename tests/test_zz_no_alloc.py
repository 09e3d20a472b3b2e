"""speckv_scores_noalloc (the scoring entry point with the library's fixed
per-GPU scratch instead of a caller workspace) against speckv_scores through
the C ABI: two calls in a row, the second on a smaller problem (the scratch
keeps the first call's contents), each bit-identical to the workspace form
and so within the score tolerance of the oracle; a problem larger than the
scratch is refused before anything is launched."""
import numpy as np
import pytest
import torch

import attention_importance_scoring_amd as skv
from attention_importance_scoring_amd import workloads as wl

from gpu_helpers import shape_of, workspace

pytestmark = pytest.mark.gpu


def _both(cfg, seed, n_layers=None):
    inp = wl.speckv_inputs(cfg, seed, "cuda", layers=range(n_layers or cfg.n_layers))
    L, H = inp["q_obs"].shape[0], cfg.n_kv_heads
    shape = shape_of(cfg, kv_head_stride=inp["kv_head_stride"], n_layers=L)
    ref = torch.full((L, H, cfg.n_pre), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full_like(ref, float("nan"))
    skv.speckv_scores(shape, inp["q_obs"], inp["k_buf"], ref, workspace(shape, cfg.C_max))
    skv.speckv_scores_noalloc(shape, inp["q_obs"], inp["k_buf"], got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_workspace_form_twice_second_smaller(gpu_lib):
    big = wl.QWEN32B_64K  # 16 of its 64 layers: about 36 MB of scratch
    print(f"\n[case] noalloc 1: {big.name}, 16 layers", flush=True)
    ref, got = _both(big, 3, n_layers=16)
    assert torch.isfinite(ref).all()
    assert torch.equal(got, ref), "scratch form differs from the workspace form (first call)"
    np.testing.assert_allclose(got.double().sum(-1).cpu().numpy(), big.G * big.n_obs, rtol=1e-4)
    small = wl.reduced(wl.LLAMA8B_16K, n_layers=3, n_in=5000 + 37, n_window=21, n_lookahead=11, C_max=300)
    print(f"[case] noalloc 2: {small.n_layers} layers, n_in={small.n_in} (smaller; stale scratch)", flush=True)
    ref2, got2 = _both(small, 5)
    assert torch.isfinite(ref2).all()
    assert torch.equal(got2, ref2), "scratch form differs from the workspace form (second, smaller call)"


def test_noalloc_refuses_problems_beyond_the_scratch(gpu_lib):
    cfg = wl.QWEN32B_64K
    shape = shape_of(cfg)
    q = torch.empty((cfg.n_layers, cfg.n_q_heads, cfg.n_obs, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((cfg.n_layers, cfg.n_kv_heads, cfg.n_in * cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    s = torch.empty((cfg.n_layers, cfg.n_kv_heads, cfg.n_pre), dtype=torch.float32, device="cuda")
    with pytest.raises(skv.SpecKVError) as e:
        skv.speckv_scores_noalloc(shape, q, k, s)
    assert e.value.status == 5  # SKV_ERR_WORKSPACE
