"""GPU parity at the full workload sizes, in the launch configuration that
bench.py times (all layers of the 16K Llama-shaped and the 64K Qwen-shaped
workloads in one call per entry point; the 128K in-place workload one layer
per call; the SpecPC draft stack in one call).

Every (layer, KV head) unit of the 16K, 64K and 128K workloads is compared
with the fp64 oracle element by element (scores within the tolerance; kept
sets exact against the rule on the GPU's own pooled scores and equal to the
oracle's up to ties within the tolerance; compacted rows bit-exact), the
oracle spread over a pool of single-threaded worker processes (about 1.3 s
of one core per 64K unit).  Properties that hold at any size (non-negative
finite scores totalling G * n_obs per head, kept lists ascending with the
window at the tail) are checked too.  The SpecPC stack is checked in full.
The variant launches (max aggregation, one kept set per query head) compare
sampled units and check the invariants on all.
"""
import numpy as np
import pytest
import torch

import attention_importance_scoring_amd as skv
import oracle
from attention_importance_scoring_amd import workloads as wl

from gpu_helpers import (assert_compacted, assert_kept_matches, assert_scores_close, check_every_unit_against_oracle,
                         np64, shape_of, workspace)

pytestmark = pytest.mark.gpu


def _check_every_unit(scores, pooled, kept, cfg):
    """Properties of every unit's outputs (host copies, fp32 from the GPU)."""
    sc = scores.astype(np.float64)
    assert np.isfinite(sc).all() and (sc >= 0).all()
    np.testing.assert_allclose(sc.sum(-1), cfg.G * cfg.n_obs, rtol=1e-4)
    n_top = min(cfg.C_max, cfg.n_pre)
    flat_kept = kept.reshape(-1, kept.shape[-1])
    flat_pooled = pooled.reshape(-1, pooled.shape[-1]).astype(np.float64)
    window = np.arange(cfg.n_pre, cfg.n_in)
    for u in range(flat_kept.shape[0]):
        kg = flat_kept[u]
        assert (np.diff(kg) > 0).all(), f"unit {u}: kept list not strictly ascending"
        assert (kg[n_top:] == window).all(), f"unit {u}: window keys missing"
        exact = oracle.select_kept(flat_pooled[u], cfg.C_max, cfg.n_window)
        assert (kg == exact).all(), f"unit {u}: selection differs from the rule on the GPU's own pooled scores"


def _check_sampled_units(scores, pooled, kept, q_obs, k, cfg, units):
    scale = oracle.default_scale(cfg.head_dim)
    G = cfg.G
    for layer, h in units:
        print(f"[unit] layer {layer} KV head {h}", flush=True)
        want = oracle.head_scores(np64(q_obs[layer, h * G:(h + 1) * G]), np64(k[layer, h])[:cfg.n_pre], scale)
        assert_scores_close(scores[layer, h], want, G, cfg.n_obs, f"scores[{layer},{h}]")
        pooled_o = oracle.pool1d(want, cfg.pool_kernel, "max")
        assert_kept_matches(kept[layer, h][None], pooled[layer, h][None], pooled_o[None], cfg.C_max, cfg.n_window,
                            f"kept[{layer},{h}]")


def test_qwen32b_shape_64k_all_layers_one_call():
    cfg = wl.QWEN32B_64K
    print(f"\n[case] {cfg.name}: 64 layers in one call, n_in={cfg.n_in}, seed 3 on the GPU", flush=True)
    inp = wl.speckv_inputs(cfg, 3, "cuda")  # the inputs bench.py times
    L, H, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    shape = shape_of(cfg, kv_head_stride=inp["kv_head_stride"])
    ws = workspace(shape, cfg.C_max)
    n_keep = skv.speckv_n_keep(shape, cfg.C_max)
    scores = torch.full((L, H, cfg.n_pre), float("nan"), dtype=torch.float32, device="cuda")
    pooled = torch.full_like(scores, float("nan"))
    kept = torch.full((L, H, n_keep), -1, dtype=torch.int32, device="cuda")
    kc = torch.empty((L, H, n_keep, d), dtype=inp["k"].dtype, device="cuda")
    vc = torch.empty_like(kc)
    skv.speckv_scores(shape, inp["q_obs"], inp["k_buf"], scores, ws)
    skv.speckv_select(shape, scores, cfg.C_max, skv.SKV_POOL_MAX, cfg.pool_kernel, kept, pooled, ws)
    skv.speckv_compact(shape, inp["k_buf"], inp["v_buf"], kept, n_keep, kc, vc, ws)
    torch.cuda.synchronize()
    assert_compacted(kc, vc, inp["k"], inp["v"], kept)
    sc, pl, kp = scores.cpu().numpy(), pooled.cpu().numpy(), kept.cpu().numpy()
    _check_every_unit(sc, pl, kp, cfg)
    check_every_unit_against_oracle(sc, pl, kp, inp["q_obs"], inp["k"], cfg, label=cfg.name)


def test_llama8b_shape_16k_all_layers_one_call():
    cfg = wl.LLAMA8B_16K
    print(f"\n[case] {cfg.name}: 32 layers in one call, n_in={cfg.n_in}, seed 3 on the GPU", flush=True)
    inp = wl.speckv_inputs(cfg, 3, "cuda")  # the inputs bench.py times
    L, H, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    shape = shape_of(cfg, kv_head_stride=inp["kv_head_stride"])
    ws = workspace(shape, cfg.C_max)
    n_keep = skv.speckv_n_keep(shape, cfg.C_max)
    scores = torch.full((L, H, cfg.n_pre), float("nan"), dtype=torch.float32, device="cuda")
    pooled = torch.full_like(scores, float("nan"))
    kept = torch.full((L, H, n_keep), -1, dtype=torch.int32, device="cuda")
    kc = torch.empty((L, H, n_keep, d), dtype=inp["k"].dtype, device="cuda")
    vc = torch.empty_like(kc)
    skv.speckv_scores(shape, inp["q_obs"], inp["k_buf"], scores, ws)
    skv.speckv_select(shape, scores, cfg.C_max, skv.SKV_POOL_MAX, cfg.pool_kernel, kept, pooled, ws)
    skv.speckv_compact(shape, inp["k_buf"], inp["v_buf"], kept, n_keep, kc, vc, ws)
    torch.cuda.synchronize()
    assert_compacted(kc, vc, inp["k"], inp["v"], kept)
    sc, pl, kp = scores.cpu().numpy(), pooled.cpu().numpy(), kept.cpu().numpy()
    _check_every_unit(sc, pl, kp, cfg)
    check_every_unit_against_oracle(sc, pl, kp, inp["q_obs"], inp["k"], cfg, label=cfg.name)


@pytest.mark.parametrize("first", [0, 16], ids=["layers-0-15", "layers-16-31"])
def test_llama8b_shape_128k_in_place_one_layer_per_call(first):
    cfg = wl.LLAMA8B_128K_INPLACE
    layers = list(range(first, first + 16))
    n = len(layers)
    print(f"\n[case] {cfg.name}: layers {layers[0]}..{layers[-1]} one per call, in place, n_in={cfg.n_in}",
          flush=True)
    inp = wl.speckv_inputs(cfg, 3, "cuda", layers=layers)  # the layers of the inputs bench.py times
    H, d = cfg.n_kv_heads, cfg.head_dim
    shape = shape_of(cfg, kv_head_stride=inp["kv_head_stride"], n_layers=1)
    ws = workspace(shape, cfg.C_max)
    n_keep = skv.speckv_n_keep(shape, cfg.C_max)
    k0, v0 = inp["k"].clone(), inp["v"].clone()
    scores = torch.full((n, H, cfg.n_pre), float("nan"), dtype=torch.float32, device="cuda")
    pooled = torch.full_like(scores, float("nan"))
    kept = torch.full((n, H, n_keep), -1, dtype=torch.int32, device="cuda")
    for i in range(n):
        sl = slice(i, i + 1)
        skv.speckv_scores(shape, inp["q_obs"][sl], inp["k_buf"][sl], scores[sl], ws)
        skv.speckv_select(shape, scores[sl], cfg.C_max, skv.SKV_POOL_MAX, cfg.pool_kernel, kept[sl], pooled[sl], ws)
        skv.speckv_compact(shape, inp["k_buf"][sl], inp["v_buf"][sl], kept[sl], n_keep, inp["k_buf"][sl],
                           inp["v_buf"][sl], ws)
    torch.cuda.synchronize()
    k_c = inp["k_buf"][:, :, :n_keep * d].unflatten(2, (n_keep, d))
    v_c = inp["v_buf"][:, :, :n_keep * d].unflatten(2, (n_keep, d))
    assert_compacted(k_c, v_c, k0, v0, kept)
    sc, pl, kp = scores.cpu().numpy(), pooled.cpu().numpy(), kept.cpu().numpy()
    red = wl.reduced(cfg, n_layers=n)
    _check_every_unit(sc, pl, kp, red)
    check_every_unit_against_oracle(sc, pl, kp, inp["q_obs"], k0, red, layer_ids=layers, label=cfg.name)


def test_specpc_draft_32k_full_stack_one_call():
    cfg = wl.SPECPC_DRAFT_32K
    print(f"\n[case] {cfg.name}: {cfg.n_layers} layers (l_skip {cfg.l_skip}), n_in={cfg.n_in}, W={cfg.window}",
          flush=True)
    inp = wl.specpc_inputs(cfg, 5, "cuda")  # the inputs bench.py times
    dt = skv.SKV_BF16
    shape = skv.make_shape(cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_in, cfg.window,
                           cfg.n_lookahead, dt)
    sel = skv.make_shape(1, 1, 1, cfg.head_dim, cfg.n_in, 0, 0, dt)
    ws = workspace(shape, cfg.k_top)
    ts = torch.full((cfg.n_in,), float("nan"), dtype=torch.float32, device="cuda")
    pooled = torch.empty_like(ts)
    kept = torch.full((cfg.k_top,), -1, dtype=torch.int32, device="cuda")
    skv.specpc_token_scores(shape, cfg.l_skip, inp["q_win"], inp["k"], None, ts, ws)
    skv.speckv_select(sel, ts, cfg.k_top, skv.SKV_POOL_MAX, cfg.pool_kernel, kept, pooled, ws)
    torch.cuda.synchronize()
    print("[oracle] full draft stack on the host", flush=True)
    want = oracle.specpc_token_scores(np64(inp["q_win"]), np64(inp["k"]), cfg.l_skip, None)
    assert_scores_close(ts.cpu().numpy(), want, cfg.G, cfg.window, "token scores")
    pooled_o = oracle.pool1d(want, cfg.pool_kernel, "max")
    assert_kept_matches(kept.cpu().numpy()[None], pooled.cpu().numpy()[None], pooled_o[None], cfg.k_top, 0, "tokens")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_many_long_units_four_key_tiles_per_wave(dtype, d):
    # 768 units of 16K keys: every block walks at least 16 groups of resident
    # keys, which is where the planner holds four key tiles per wave.
    cfg = wl.reduced(wl.LLAMA8B_16K, n_layers=96, n_q_heads=8, n_kv_heads=8, head_dim=d, dtype=dtype,
                     n_in=16384 + 8, n_window=8, n_lookahead=4, C_max=200)
    print(f"\n[case] {cfg.n_layers * cfg.n_kv_heads} units, {dtype} d={d}, n_in={cfg.n_in}", flush=True)
    inp = wl.speckv_inputs(cfg, 31, "cuda")
    L, H = cfg.n_layers, cfg.n_kv_heads
    shape = shape_of(cfg, kv_head_stride=inp["kv_head_stride"])
    ws = workspace(shape, cfg.C_max)
    n_keep = skv.speckv_n_keep(shape, cfg.C_max)
    scores = torch.full((L, H, cfg.n_pre), float("nan"), dtype=torch.float32, device="cuda")
    pooled = torch.full_like(scores, float("nan"))
    kept = torch.full((L, H, n_keep), -1, dtype=torch.int32, device="cuda")
    skv.speckv_scores(shape, inp["q_obs"], inp["k_buf"], scores, ws)
    skv.speckv_select(shape, scores, cfg.C_max, skv.SKV_POOL_MAX, cfg.pool_kernel, kept, pooled, ws)
    torch.cuda.synchronize()
    sc, pl, kp = scores.cpu().numpy(), pooled.cpu().numpy(), kept.cpu().numpy()
    _check_every_unit(sc, pl, kp, cfg)
    _check_sampled_units(sc, pl, kp, inp["q_obs"], inp["k"], cfg, [(0, 0), (47, 3), (95, 7)])


@pytest.mark.parametrize("aggregation,per_query_head", [("max", False), ("sum", True)],
                         ids=["max-per-kv-head", "sum-per-query-head"])
def test_qwen32b_shape_64k_variants_one_call(aggregation, per_query_head):
    # the bench's --aggregation max and --per-query-head launches on the same inputs
    cfg = wl.QWEN32B_64K
    print(f"\n[case] {cfg.name} {aggregation} per_query_head={per_query_head}: 64 layers in one call", flush=True)
    inp = wl.speckv_inputs(cfg, 3, "cuda")
    L, Hq, Hkv, d, G = cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.G
    H = Hq if per_query_head else Hkv
    shape = skv.make_shape(L, Hq, Hkv, d, cfg.n_in, cfg.n_window, cfg.n_lookahead, skv.SKV_BF16,
                           kv_head_stride=inp["kv_head_stride"],
                           aggregation=skv.SKV_AGG_MAX if aggregation == "max" else skv.SKV_AGG_SUM,
                           per_query_head=int(per_query_head))
    ws = workspace(shape, cfg.C_max)
    n_keep = skv.speckv_n_keep(shape, cfg.C_max)
    scores = torch.full((L, H, cfg.n_pre), float("nan"), dtype=torch.float32, device="cuda")
    pooled = torch.full_like(scores, float("nan"))
    kept = torch.full((L, H, n_keep), -1, dtype=torch.int32, device="cuda")
    kc = torch.empty((L, H, n_keep, d), dtype=inp["k"].dtype, device="cuda")
    vc = torch.empty_like(kc)
    skv.speckv_scores(shape, inp["q_obs"], inp["k_buf"], scores, ws)
    skv.speckv_select(shape, scores, cfg.C_max, skv.SKV_POOL_MAX, cfg.pool_kernel, kept, pooled, ws)
    skv.speckv_compact(shape, inp["k_buf"], inp["v_buf"], kept, n_keep, kc, vc, ws)
    torch.cuda.synchronize()
    # compacted rows: query head h's cache holds rows of KV head h // G
    if per_query_head:
        for g in range(G):  # query heads g, G + g, 2 G + g, ... read KV heads 0, 1, 2, ...
            assert_compacted(kc[:, g::G], vc[:, g::G], inp["k"], inp["v"], kept[:, g::G])
    else:
        assert_compacted(kc, vc, inp["k"], inp["v"], kept)
    sc = scores.cpu().numpy().astype(np.float64)
    assert np.isfinite(sc).all() and (sc >= 0).all()
    rows = cfg.n_obs * (1 if per_query_head else G)
    if aggregation == "max":
        assert (sc <= 1.0 + 1e-6).all()  # a maximum of probabilities
    else:
        np.testing.assert_allclose(sc.sum(-1), rows, rtol=1e-4)
    pl, kp = pooled.cpu().numpy(), kept.cpu().numpy()
    for u in range(0, L * H, 37):  # the selection rule on the GPU's own pooled scores, a spread of units
        layer, h = divmod(u, H)
        exact = oracle.select_kept(pl[layer, h].astype(np.float64), cfg.C_max, cfg.n_window)
        assert (kp[layer, h] == exact).all(), f"unit {u}: selection differs from the rule on its own scores"
    scale = oracle.default_scale(d)
    for layer, h in [(0, 0), (29, 3), (63, H - 1)]:
        print(f"[unit] layer {layer} head {h}", flush=True)
        q = inp["q_obs"][layer, h:h + 1] if per_query_head else inp["q_obs"][layer, h * G:(h + 1) * G]
        kvh = h // G if per_query_head else h
        want = oracle.head_scores(np64(q), np64(inp["k"][layer, kvh])[:cfg.n_pre], scale, aggregation)
        assert_scores_close(sc[layer, h], want, 1 if per_query_head else G, cfg.n_obs, f"scores[{layer},{h}]")
        assert_kept_matches(kp[layer, h][None], pl[layer, h][None], oracle.pool1d(want, cfg.pool_kernel, "max")[None],
                            cfg.C_max, cfg.n_window, f"kept[{layer},{h}]")
