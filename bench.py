"""Throughput of the SpecKV scoring + selection + compaction path on one MI355X.

One step = speckv_scores + speckv_select + speckv_compact over every layer
and KV head of the workload (default: the Qwen2.5-32B-shaped 64K-token
workload: 64 layers, 40 query / 8 KV heads, head_dim 128, bf16, 32 window +
128 lookahead queries, C_max 256, max-pool 7).  Inputs are synthetic, seeded
and resident in HBM before timing starts.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

--gpus N with N > 1 is refused: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "keys scored+compacted/sec and % of HBM/MFMA roofline at n_in=64K, 32B shape"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# v_exp_f32: 256 CUs x 32 exponentials per clock (one wave64 instruction per 8 cycles on each of the 4 SIMDs)
# x 2.4 GHz; the peak-check program measures 17.4 T/s, about 9 cycles per instruction.
PEAK_EXP_TPS = 256 * 32 * 2.4e9 / 1e12
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="qwen32b_shape_64k",
                   choices=["qwen32b_shape_64k", "llama8b_shape_16k", "llama8b_shape_128k_inplace", "specpc_draft_32k",
                            "speckv_pc_cascade_32k", "decode_qwen32b_shape_64k"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--aggregation", choices=["sum", "max"], default="sum",
                   help="SpecKV: aggregate the observation rows' probabilities by sum (default) or max")
    p.add_argument("--per-query-head", action="store_true",
                   help="SpecKV: one kept set (and compacted cache) per query head instead of per KV head")
    p.add_argument("--n-lookahead", type=int, default=None,
                   help="draft lookahead tokens (default: the workload's).  SpecKV: 0 scores with the window "
                        "queries only; SpecPC: > 1 puts draft rows at the end of the window")
    p.add_argument("--pool-kernel", type=int, default=None,
                   help="SpecKV: max-pool width before selection (odd; 1 = no pooling; default: the workload's)")
    p.add_argument("--decode-cache", choices=["both", "compacted", "full"], default="both",
                   help="decode workload: time decode over the compacted cache, the full cache, or both")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration runs)")
    p.add_argument("--cascade-path", choices=["rows", "gather"], default="rows",
                   help="cascade: SpecKV through the kept-token list, or on a gathered copy of the target cache")
    p.add_argument("--seed", type=int, default=0)
    return p.parse_args()


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def speckv_cpu_baseline(cfg, inp, budget_s=12.0):
    """The fp64 oracle (scores, pooling, selection, compaction) on whole
    (layer, KV head) units of the same workload, until ~budget_s of work."""
    import numpy as np
    import torch
    import oracle
    from attention_importance_scoring_amd import workloads as wl
    G = cfg.G
    done, keys, t_total = 0, 0, 0.0
    L = inp["q_obs"].shape[0]
    units = [(l, h) for l in range(L) for h in range(cfg.n_kv_heads)]
    rng = np.random.default_rng(0)
    order = rng.permutation(len(units))
    for idx in order:
        l, h = units[idx]
        q = wl.to_numpy_f64(inp["q_obs"][l, h * G:(h + 1) * G])
        k = wl.to_numpy_f64(inp["k"][l, h])
        v = inp["v"][l, h].cpu()
        v_raw = v.view(torch.int16).numpy() if v.dtype == torch.bfloat16 else v.numpy()  # bit copy
        t0 = time.perf_counter()
        s = oracle.head_scores(q, k[:cfg.n_pre], oracle.default_scale(cfg.head_dim))
        pooled = oracle.pool1d(s, cfg.pool_kernel, "max")
        kept = oracle.select_kept(pooled, cfg.C_max, cfg.n_window)
        oracle.compact_rows(k, kept)
        oracle.compact_rows(v_raw, kept)
        t_total += time.perf_counter() - t0
        done += 1
        keys += cfg.n_in
        if t_total >= budget_s:
            break
    return {"value": keys / t_total, "unit": "keys/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{done} of {len(units)} (layer, KV head) units of the same workload, {keys} keys, "
                      f"{t_total:.1f} s of fp64 NumPy"}


def decode_cpu_baseline(cfg, inp, cache, budget_s=10.0):
    """The fp64 decode-attention oracle on whole (layer, KV head) units of
    the same caches (the compacted 288-row one unless only the full cache is
    benchmarked), until ~budget_s of work; scaled to all-layer decode steps/s."""
    import numpy as np
    import oracle
    from attention_importance_scoring_amd import workloads as wl
    G, d = cfg.G, cfg.head_dim
    L, H = cfg.n_layers, cfg.n_kv_heads
    n_rows = cfg.n_keep if cache != "full" else cfg.n_in
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, G, d))
    order = rng.permutation(L * H)
    units = []  # host copies of up to 64 units, visited round-robin until the budget is spent
    for idx in order[:64]:
        layer, h = divmod(int(idx), H)
        units.append((wl.to_numpy_f64(inp["k"][layer:layer + 1, h:h + 1, :n_rows]),
                      wl.to_numpy_f64(inp["v"][layer:layer + 1, h:h + 1, :n_rows])))
    done, t_total = 0, 0.0
    while t_total < budget_s:
        k, v = units[done % len(units)]
        t0 = time.perf_counter()
        oracle.decode_attention(q, k, v)
        t_total += time.perf_counter() - t0
        done += 1
    per_step = t_total / done * (L * H)
    return {"value": 1.0 / per_step, "unit": "decode steps/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{done} unit decodes over {len(units)} distinct (layer, KV head) units of {n_rows} rows "
                      f"(the first rows of the full cache stand in for the compacted ones), {t_total:.1f} s of "
                      f"fp64 NumPy, scaled to all {L * H} units of one decode step"}


def _specpc_oracle_time(cfg, inp, budget_s):
    """Seconds per step of the fp64 oracle's SpecPC token scores and selection:
    one used layer at a time (all its query heads) until ~budget_s, scaled
    to every used layer.  Returns (seconds, layers timed, used layers,
    selection seconds, kept tokens)."""
    import oracle
    from attention_importance_scoring_amd import workloads as wl
    used = list(range(cfg.l_skip, cfg.n_layers))
    done, t_layers, scores = 0, 0.0, None
    for layer in used:
        q = wl.to_numpy_f64(inp["q_win"][layer:layer + 1])
        k = wl.to_numpy_f64(inp["k"][layer:layer + 1])
        t0 = time.perf_counter()
        scores = oracle.specpc_token_scores(q, k, 0, n_in=cfg.n_in)
        t_layers += time.perf_counter() - t0
        done += 1
        if t_layers >= budget_s:
            break
    t0 = time.perf_counter()
    tokens, _ = oracle.specpc_select(scores, cfg.k_top, "max", cfg.pool_kernel)
    t_sel = time.perf_counter() - t0
    return t_layers / done * len(used) + t_sel, done, len(used), t_sel, tokens


def specpc_cpu_baseline(cfg, inp, budget_s=12.0):
    """The fp64 oracle's SpecPC token scores one used layer at a time (all
    its query heads), until ~budget_s of work, scaled to every used layer,
    plus its pooling and selection once."""
    per_step, done, n_used, t_sel, _ = _specpc_oracle_time(cfg, inp, budget_s)
    return {"value": cfg.n_in / per_step, "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{done} of {n_used} used layers ({done * cfg.n_q_heads} causal window maps of "
                      f"{cfg.window} x {cfg.n_keys}), about {budget_s:.0f} s of fp64 NumPy, scaled to all used "
                      f"layers, plus pooling and selection ({t_sel:.2f} s)"}


def cascade_cpu_baseline(cc, inp, budget_s=12.0):
    """The fp64 oracle's cascade: SpecPC on the draft as in
    specpc_cpu_baseline (half the budget), then SpecKV on the compressed
    prompt over whole (layer, KV head) units of the target, gathering the
    kept tokens' rows, scoring, pooling, selecting and compacting (the
    other half), scaled to all units."""
    import numpy as np
    import torch
    import oracle
    from attention_importance_scoring_amd import workloads as wl
    dr, tg = cc.draft, cc.target
    pc_s, pc_done, pc_used, _, tokens = _specpc_oracle_time(dr, inp["draft"], budget_s / 2)
    t_in = inp["target"]
    G, n_tok = tg.n_q_heads // tg.n_kv_heads, len(tokens)
    units = [(l, h) for l in range(tg.n_layers) for h in range(tg.n_kv_heads)]
    order = np.random.default_rng(0).permutation(len(units))
    done, t_units = 0, 0.0
    for idx in order:
        l, h = units[idx]
        q = wl.to_numpy_f64(t_in["q_obs"][l, h * G:(h + 1) * G])
        k = wl.to_numpy_f64(t_in["k"][l, h])
        v = t_in["v"][l, h].cpu()
        v_raw = v.view(torch.int16).numpy() if v.dtype == torch.bfloat16 else v.numpy()  # bit copy
        t0 = time.perf_counter()
        k_c, v_c = k[tokens], v_raw[tokens]
        s = oracle.head_scores(q, k_c[:n_tok - tg.n_window], oracle.default_scale(tg.head_dim))
        kept = oracle.select_kept(oracle.pool1d(s, tg.pool_kernel, "max"), tg.C_max, tg.n_window)
        oracle.compact_rows(k_c, kept)
        oracle.compact_rows(v_c, kept)
        t_units += time.perf_counter() - t0
        done += 1
        if t_units >= budget_s / 2:
            break
    per_step = pc_s + t_units / done * len(units)
    return {"value": dr.n_in / per_step, "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"SpecPC: {pc_done} of {pc_used} used draft layers, scaled to all; SpecKV on the "
                      f"{n_tok}-token prompt: {done} of {len(units)} (layer, KV head) units, scaled to all; "
                      f"about {budget_s:.0f} s of fp64 NumPy in total"}


def traffic_for(kernel: str, workload: str, summary: str):
    """HBM bytes per launch of `kernel` (calibrated FETCH_SIZE + WRITE_SIZE)
    from the committed counter summary profiles/<summary>, or None when it
    is absent, covers another workload or was taken on different kernel
    sources."""
    from attention_importance_scoring_amd.counters import kernel_source_hash
    try:
        with open(os.path.join(PROFILES, summary)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    for name, k in t.get("kernels", {}).items():
        if name.startswith(kernel + "_kernel"):
            return k.get("hbm_bytes_per_launch")
    return None


def bench_speckv(args, cfg, torch, skv, wl):
    from_layers = None
    dev = "cuda"
    if args.n_lookahead is not None:
        cfg = wl.reduced(cfg, n_lookahead=args.n_lookahead)
    if args.pool_kernel is not None:
        cfg = wl.reduced(cfg, pool_kernel=args.pool_kernel)
    t0 = time.perf_counter()
    inp = wl.speckv_inputs(cfg, seed=args.seed or 3, device=dev, layers=from_layers)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    L, Hkv, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    H = cfg.n_q_heads if args.per_query_head else Hkv  # heads that get their own kept set
    dt = skv.SKV_F32 if cfg.dtype == "f32" else skv.SKV_BF16
    per_layer = cfg.in_place  # the in-place workload keeps one layer's cache per call
    if per_layer and args.per_query_head:
        raise SystemExit("per-query-head caches are compacted out of place; the in-place workload does not take it")
    call_layers = 1 if per_layer else L
    shape = skv.make_shape(call_layers, cfg.n_q_heads, Hkv, d, cfg.n_in, cfg.n_window, cfg.n_lookahead, dt,
                           aggregation=skv.SKV_AGG_MAX if args.aggregation == "max" else skv.SKV_AGG_SUM,
                           per_query_head=int(args.per_query_head))
    ws = torch.empty(skv.speckv_workspace_bytes(shape, cfg.C_max), dtype=torch.uint8, device=dev)
    n_keep = skv.speckv_n_keep(shape, cfg.C_max)
    scores = torch.empty((L, H, cfg.n_pre), dtype=torch.float32, device=dev)
    pooled = torch.empty_like(scores)
    kept = torch.empty((L, H, n_keep), dtype=torch.int32, device=dev)
    kc = torch.empty((L, H, n_keep, d), dtype=inp["k"].dtype, device=dev) if not per_layer else None
    vc = torch.empty_like(kc) if kc is not None else None
    stream = torch.cuda.current_stream()
    kbuf, vbuf = inp["k_buf"], inp["v_buf"]

    def step():
        if not per_layer:
            skv.speckv_scores(shape, inp["q_obs"], kbuf, scores, ws, stream)
            skv.speckv_select(shape, scores, cfg.C_max, skv.SKV_POOL_MAX, cfg.pool_kernel, kept, pooled, ws, stream)
            skv.speckv_compact(shape, kbuf, vbuf, kept, n_keep, kc, vc, ws, stream)
        else:
            for layer in range(L):
                skv.speckv_scores(shape, inp["q_obs"][layer:layer + 1], kbuf[layer:layer + 1], scores[layer:layer + 1],
                                  ws, stream)
                skv.speckv_select(shape, scores[layer:layer + 1], cfg.C_max, skv.SKV_POOL_MAX, cfg.pool_kernel,
                                  kept[layer:layer + 1], pooled[layer:layer + 1], ws, stream)
                skv.speckv_compact(shape, kbuf[layer:layer + 1], vbuf[layer:layer + 1], kept[layer:layer + 1], n_keep,
                                   kbuf[layer:layer + 1], vbuf[layer:layer + 1], ws, stream)

    print(f"[bench] inputs ready ({gen_s:.1f} s); warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    skv.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    prof = skv.profile_read()
    skv.profile_enable(False)
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    keys = cfg.keys_per_call  # KV pairs scored and compacted (each query head's copy counted once)
    flops_per_pass = 2.0 * cfg.n_obs * cfg.n_q_heads * L * cfg.n_pre * d  # one Q_obs K^T over every head
    default_variant = (args.aggregation == "sum" and not args.per_query_head and args.n_lookahead is None
                       and args.pool_kernel is None)
    kern = {name: {"launches": n, "avg_ms": t / max(n, 1), "ms_per_step": t / args.steps} for name, (n, t) in prof.items()}
    # dominant kernel: the longer of the two scoring passes (each computes one Q_obs K^T)
    dom = max(("score_pass1", "score_pass2"), key=lambda k: kern[k]["ms_per_step"])
    launches_per_step = kern[dom]["launches"] / args.steps
    flops_per_launch = flops_per_pass / launches_per_step
    avg_s = kern[dom]["avg_ms"] * 1e-3
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    achieved = flops_per_launch / avg_s / 1e12
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic_for(dom, cfg.name, f"speckv_kernels_{cfg.name}_traffic.json") if default_variant else None}
    # whole path against the MFMA roofline: one Q_obs K^T is the method's algorithmic work
    path_frac = (flops_per_pass / (ms * 1e-3) / 1e12) / peak
    out = {
        "metric": METRIC, "value": keys / (ms * 1e-3), "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "n_layers": L, "n_q_heads": cfg.n_q_heads, "n_kv_heads": Hkv, "head_dim": d,
                   "n_in": cfg.n_in, "n_window": cfg.n_window, "n_lookahead": cfg.n_lookahead, "C_max": cfg.C_max,
                   "pool_kernel": cfg.pool_kernel, "in_place": cfg.in_place, "keys_per_step": keys,
                   "aggregation": args.aggregation, "per_query_head": bool(args.per_query_head)},
        "roofline": roof,
        "path_mfma_frac": round(path_frac, 4),
        "kernels": {k: {"avg_ms": round(v["avg_ms"], 4), "ms_per_step": round(v["ms_per_step"], 4)}
                    for k, v in kern.items()},
    }
    return out, inp


def bench_specpc(args, cfg, torch, skv, wl):
    dev = "cuda"
    if args.n_lookahead is not None:
        cfg = wl.reduced(cfg, n_lookahead=args.n_lookahead)
    inp = wl.specpc_inputs(cfg, seed=args.seed or 5, device=dev)
    dt = skv.SKV_F32 if cfg.dtype == "f32" else skv.SKV_BF16
    shape = skv.make_shape(cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_in, cfg.window,
                           cfg.n_lookahead, dt, kv_head_stride=cfg.n_keys * cfg.head_dim)
    sel = skv.make_shape(1, 1, 1, cfg.head_dim, cfg.n_in, 0, 0, dt)
    ws = torch.empty(skv.speckv_workspace_bytes(shape, 0), dtype=torch.uint8, device=dev)
    ts = torch.empty(cfg.n_in, dtype=torch.float32, device=dev)
    pooled = torch.empty_like(ts)
    kept = torch.empty(cfg.k_top, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        skv.specpc_token_scores(shape, cfg.l_skip, inp["q_win"], inp["k"], None, ts, ws, stream)
        skv.speckv_select(sel, ts, cfg.k_top, skv.SKV_POOL_MAX, cfg.pool_kernel, kept, pooled, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    skv.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    prof = skv.profile_read()
    skv.profile_enable(False)
    kern = {name: {"avg_ms": round(t / max(n, 1), 4), "ms_per_step": round(t / args.steps, 4)}
            for name, (n, t) in prof.items()}
    maps = (cfg.n_layers - cfg.l_skip) * cfg.n_q_heads
    elems = maps * sum(min(cfg.n_keys, cfg.n_keys - cfg.window + i + 1) for i in range(cfg.window))
    exps_per_s = 2 * elems / (ms * 1e-3)  # two passes, one exp per (row, visible key) each
    # Both passes evaluate one exponential per (map, window row, visible key): the exp roofline of the longer one.
    dom = max(("score_pass1", "specpc_pass2"), key=lambda k: kern.get(k, {}).get("avg_ms", 0.0))
    achieved = elems / (kern[dom]["avg_ms"] * 1e-3) / 1e12
    default_cfg = args.n_lookahead is None
    roof = {"kernel": dom, "bound": "alu", "achieved": round(achieved, 3), "peak": round(PEAK_EXP_TPS, 2),
            "unit": "T exp/s", "frac": round(achieved / PEAK_EXP_TPS, 4),
            "traffic": traffic_for(dom, cfg.name, f"specpc_kernels_{cfg.name}_traffic.json") if default_cfg else None}
    return {
        "metric": "SpecPC tokens scored+selected/sec (draft attention stack)", "value": cfg.n_in / (ms * 1e-3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "n_layers": cfg.n_layers, "l_skip": cfg.l_skip, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "n_in": cfg.n_in, "window": cfg.window,
                   "n_lookahead": cfg.n_lookahead, "k_top": cfg.k_top},
        "roofline": roof, "exp_rate_per_s": exps_per_s, "kernels": kern,
    }, inp


def bench_cascade(args, cc, torch, skv, wl):
    """SpecKV-PC: SpecPC token scores + selection on the draft stack, then
    SpecKV scores, selection and compaction over the compressed prompt, all
    on one stream.  Path "rows" (default): SpecKV reads the target cache
    through the kept-token list; "gather": the target cache is first gathered
    at the kept tokens."""
    dev = "cuda"
    inp = wl.cascade_inputs(cc, seed=args.seed or 5, device=dev)
    torch.cuda.synchronize()
    dr, st2, tg = cc.draft, cc.stage2, inp["target"]
    dt = skv.SKV_F32 if dr.dtype == "f32" else skv.SKV_BF16
    pc_shape = skv.make_shape(dr.n_layers, dr.n_q_heads, dr.n_kv_heads, dr.head_dim, dr.n_in, dr.window,
                              dr.n_lookahead, dt)
    sel_shape = skv.make_shape(1, 1, 1, dr.head_dim, dr.n_in, 0, 0, dt)
    full_shape = skv.make_shape(cc.target.n_layers, cc.target.n_q_heads, cc.target.n_kv_heads, cc.target.head_dim,
                                cc.target.n_in, cc.target.n_window, cc.target.n_lookahead, skv.SKV_BF16,
                                kv_head_stride=tg["kv_head_stride"])
    s2_shape = skv.make_shape(st2.n_layers, st2.n_q_heads, st2.n_kv_heads, st2.head_dim, st2.n_in, st2.n_window,
                              st2.n_lookahead, skv.SKV_BF16)
    rows_shape = skv.make_shape(st2.n_layers, st2.n_q_heads, st2.n_kv_heads, st2.head_dim, st2.n_in, st2.n_window,
                                st2.n_lookahead, skv.SKV_BF16, kv_head_stride=tg["kv_head_stride"])
    use_rows = args.cascade_path == "rows"
    ws = torch.empty(skv.speckv_workspace_bytes(pc_shape, dr.k_top), dtype=torch.uint8, device=dev)
    ws2 = torch.empty(skv.speckv_workspace_bytes(s2_shape, st2.C_max), dtype=torch.uint8, device=dev)
    L, H, d, n_tok = st2.n_layers, st2.n_kv_heads, st2.head_dim, dr.k_top
    ts = torch.empty(dr.n_in, dtype=torch.float32, device=dev)
    ts_pooled = torch.empty_like(ts)
    tokens = torch.empty(n_tok, dtype=torch.int32, device=dev)
    k_tok = None if use_rows else torch.empty((L, H, n_tok, d), dtype=tg["k"].dtype, device=dev)
    v_tok = None if use_rows else torch.empty_like(k_tok)
    n_keep = skv.speckv_n_keep(s2_shape, st2.C_max)
    scores = torch.empty((L, H, st2.n_pre), dtype=torch.float32, device=dev)
    pooled = torch.empty_like(scores)
    kept = torch.empty((L, H, n_keep), dtype=torch.int32, device=dev)
    kc = torch.empty((L, H, n_keep, d), dtype=tg["k"].dtype, device=dev)
    vc = torch.empty_like(kc)
    stream = torch.cuda.current_stream()

    def step():
        skv.specpc_token_scores(pc_shape, dr.l_skip, inp["draft"]["q_win"], inp["draft"]["k"], None, ts, ws, stream)
        skv.speckv_select(sel_shape, ts, dr.k_top, skv.SKV_POOL_MAX, dr.pool_kernel, tokens, ts_pooled, ws, stream)
        if use_rows:
            skv.speckv_scores_rows(rows_shape, tg["q_obs"], tg["k_buf"], tokens, cc.target.n_in, scores, ws2, stream)
            skv.speckv_select(rows_shape, scores, st2.C_max, skv.SKV_POOL_MAX, st2.pool_kernel, kept, pooled, ws2,
                              stream)
            skv.speckv_compact_rows(rows_shape, tg["k_buf"], tg["v_buf"], tokens, cc.target.n_in, kept, n_keep, kc, vc,
                                    stream)
        else:
            skv.specpc_gather_tokens(full_shape, tg["k_buf"], tg["v_buf"], tokens, n_tok, k_tok, v_tok, stream)
            skv.speckv_scores(s2_shape, tg["q_obs"], k_tok, scores, ws2, stream)
            skv.speckv_select(s2_shape, scores, st2.C_max, skv.SKV_POOL_MAX, st2.pool_kernel, kept, pooled, ws2,
                              stream)
            skv.speckv_compact(s2_shape, k_tok, v_tok, kept, n_keep, kc, vc, ws2, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    skv.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    prof = skv.profile_read()
    skv.profile_enable(False)
    kern = {name: {"launches": n, "avg_ms": round(t / max(n, 1), 4), "ms_per_step": round(t / args.steps, 4)}
            for name, (n, t) in prof.items()}
    # The longest launch is SpecPC's pass 2 on the draft: its exp roofline, as in the SpecPC workload.
    pc_maps = (dr.n_layers - dr.l_skip) * dr.n_q_heads
    pc_elems = pc_maps * sum(min(dr.n_keys, dr.n_keys - dr.window + i + 1) for i in range(dr.window))
    pc_ach = pc_elems / (kern["specpc_pass2"]["avg_ms"] * 1e-3) / 1e12
    roof = {"kernel": "specpc_pass2", "bound": "alu", "achieved": round(pc_ach, 3), "peak": round(PEAK_EXP_TPS, 2),
            "unit": "T exp/s", "frac": round(pc_ach / PEAK_EXP_TPS, 4),
            "traffic": traffic_for("specpc_pass2", cc.name, f"cascade_kernels_{cc.name}_traffic.json")}
    # the gather moves n_tok rows of K and V per (layer, KV head) in and out
    g = kern.get("gather_tokens")
    gather_bytes = 2 * 2 * L * H * n_tok * d * 2  # K and V, read and write, bf16
    gather_gbs = gather_bytes / (g["ms_per_step"] * 1e-3) / 1e9 if g else None
    return {
        "metric": "SpecKV-PC cascade: prompt tokens compressed/sec (SpecPC to k_top tokens, SpecKV to C_max pairs)",
        "value": dr.n_in / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dr.dtype, "data": "synthetic",
        "config": {"workload": cc.name, "n_in": dr.n_in, "draft_layers": dr.n_layers, "l_skip": dr.l_skip,
                   "draft_heads": [dr.n_q_heads, dr.n_kv_heads, dr.head_dim], "window": dr.window, "k_top": n_tok,
                   "target_layers": L, "target_heads": [st2.n_q_heads, H, d], "n_window": st2.n_window,
                   "n_lookahead": st2.n_lookahead, "C_max": st2.C_max, "path": args.cascade_path},
        "gather_tokens_GBps": round(gather_gbs, 1) if gather_gbs else None,
        "roofline": roof, "kernels": kern,
    }, inp


def bench_decode(args, cfg, torch, skv, wl):
    """Decode attention for one new token per query head, all layers in one
    call, over the compacted cache that scores + select + compact produce
    (n_keep rows per KV head) and, for comparison, over the full cache
    (n_in rows).  The timed call is the compacted one; both are reported."""
    dev = "cuda"
    inp = wl.speckv_inputs(cfg, seed=args.seed or 3, device=dev)
    L, Hq, Hkv, d = cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    shape = skv.make_shape(L, Hq, Hkv, d, cfg.n_in, cfg.n_window, cfg.n_lookahead, skv.SKV_BF16)
    ws = torch.empty(skv.speckv_workspace_bytes(shape, cfg.C_max), dtype=torch.uint8, device=dev)
    n_keep = skv.speckv_n_keep(shape, cfg.C_max)
    scores = torch.empty((L, Hkv, cfg.n_pre), dtype=torch.float32, device=dev)
    kept = torch.empty((L, Hkv, n_keep), dtype=torch.int32, device=dev)
    kc = torch.empty((L, Hkv, n_keep, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    skv.speckv_scores(shape, inp["q_obs"], inp["k_buf"], scores, ws)
    skv.speckv_select(shape, scores, cfg.C_max, skv.SKV_POOL_MAX, cfg.pool_kernel, kept, None, ws)
    skv.speckv_compact(shape, inp["k_buf"], inp["v_buf"], kept, n_keep, kc, vc, ws)
    g = torch.Generator(device=dev).manual_seed(args.seed or 7)
    q = torch.randn((L, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((L, Hq, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def timed(sh, n_rows, k, v, reps):
        n_ws = skv.speckv_decode_workspace_bytes(sh, n_rows)
        w = torch.empty(n_ws, dtype=torch.uint8, device=dev) if n_ws else None
        for _ in range(args.warmup):
            skv.speckv_decode_attention(sh, n_rows, q, k, v, out, w, stream)
        torch.cuda.synchronize()
        skv.profile_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            skv.speckv_decode_attention(sh, n_rows, q, k, v, out, w, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        prof = skv.profile_read()
        skv.profile_enable(False)
        n, t = prof["decode_attention"]
        return e0.elapsed_time(e1) / reps, t / n

    def alg_bytes(n_rows):  # K and V rows read once, the queries read, the fp32 outputs written
        return L * Hkv * n_rows * d * 2 * 2 + L * Hq * d * 2 + L * Hq * d * 4

    res = {}
    if args.decode_cache in ("both", "compacted"):
        c_shape = skv.make_shape(L, Hq, Hkv, d, n_keep, 0, 0, skv.SKV_BF16)
        reps = max(args.steps, 1) * 10
        ms, kern = timed(c_shape, n_keep, kc, vc, reps)
        res["compacted"] = {"ms": round(ms, 5), "kernel_ms": round(kern, 5), "reps": reps, "rows": n_keep,
                            "GBps": round(alg_bytes(n_keep) / (kern * 1e-3) / 1e9, 1), "bytes": alg_bytes(n_keep)}
    if args.decode_cache in ("both", "full"):
        reps = max(args.steps, 1)
        ms, kern = timed(shape, cfg.n_in, inp["k_buf"], inp["v_buf"], reps)
        res["full_cache"] = {"ms": round(ms, 4), "kernel_ms": round(kern, 4), "reps": reps, "rows": cfg.n_in,
                             "GBps": round(alg_bytes(cfg.n_in) / (kern * 1e-3) / 1e9, 1),
                             "bytes": alg_bytes(cfg.n_in)}
    print(f"[bench] decode: {json.dumps(res)}", file=sys.stderr, flush=True)
    head = res.get("compacted") or res["full_cache"]
    out = {
        "metric": "decode attention over the " + ("compacted" if "compacted" in res else "full") +
                  " KV cache: layer-steps/sec (all layers, one token)",
        "value": 1e3 / head["ms"], "unit": "decode steps/s", "n_gpus": 1, "steps": head["reps"],
        "warmup": args.warmup, "ms_per_step": head["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode_" + cfg.name, "n_layers": L, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": d, "rows_compacted": n_keep, "rows_full": cfg.n_in, "cache": args.decode_cache},
    }
    if "full_cache" in res:
        f = res["full_cache"]
        out["roofline"] = {"kernel": "decode_attention (full cache)", "bound": "hbm", "achieved": f["GBps"],
                           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(f["GBps"] / PEAK_HBM_GBS, 4),
                           "traffic": traffic_for("decode_attention", "decode_" + cfg.name,
                                                  f"decode_attention_{cfg.name}_traffic.json")}
    out.update(res)
    if len(res) == 2:
        out["speedup_vs_full_cache"] = round(res["full_cache"]["ms"] / res["compacted"]["ms"], 1)
    return out, inp


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the scoring path is per-GPU work with no collectives "
              "(units are independent, so a GPU's share is the same launch over fewer layers); "
              "rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import attention_importance_scoring_amd as skv
    from attention_importance_scoring_amd import _lib
    from attention_importance_scoring_amd import workloads as wl
    _lib.load()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    cfg = wl.WORKLOADS.get(args.workload)
    if args.workload == "decode_qwen32b_shape_64k":
        cfg = wl.QWEN32B_64K
        out, inp = bench_decode(args, cfg, torch, skv, wl)
    elif args.workload in wl.CASCADES:
        out, inp = bench_cascade(args, wl.CASCADES[args.workload], torch, skv, wl)
    elif args.workload == "specpc_draft_32k":
        out, inp = bench_specpc(args, cfg, torch, skv, wl)
    else:
        out, inp = bench_speckv(args, cfg, torch, skv, wl)
    if args.calib_copy_mib:
        # plain streaming kernel of known size for counter calibration: M MiB read, M MiB written
        n = (args.calib_copy_mib << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = n * 4
    if not args.no_cpu_baseline and args.workload in wl.CASCADES:
        print("[bench] timing the fp64 oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cascade_cpu_baseline(wl.CASCADES[args.workload], inp)
    elif not args.no_cpu_baseline and args.workload == "specpc_draft_32k":
        print("[bench] timing the fp64 oracle on a sample", file=sys.stderr, flush=True)
        pc_cfg = wl.reduced(cfg, n_lookahead=args.n_lookahead) if args.n_lookahead is not None else cfg
        out["cpu_baseline"] = specpc_cpu_baseline(pc_cfg, inp)
    elif not args.no_cpu_baseline and args.workload == "decode_qwen32b_shape_64k":
        print("[bench] timing the fp64 oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = decode_cpu_baseline(cfg, inp, args.decode_cache)
    elif not args.no_cpu_baseline and args.workload in wl.WORKLOADS \
            and args.workload != "specpc_draft_32k":
        print("[bench] timing the fp64 oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = speckv_cpu_baseline(cfg, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
