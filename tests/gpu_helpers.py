"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare its outputs with the oracle under the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import attention_importance_scoring_amd as skv
from attention_importance_scoring_amd import workloads as wl

SCORE_RTOL = 1e-3  # importance scores: within 1e-3 relative


def shape_of(cfg, kv_head_stride=0, n_layers=None):
    dt = skv.SKV_F32 if cfg.dtype == "f32" else skv.SKV_BF16
    return skv.make_shape(n_layers or cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_in,
                          cfg.n_window, cfg.n_lookahead, dt, kv_head_stride=kv_head_stride)


def workspace(shape, C_max, device="cuda"):
    n = skv.speckv_workspace_bytes(shape, C_max)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def run_speckv(cfg, inp, C_max=None, pool=skv.SKV_POOL_MAX, pool_kernel=None, in_place=False, stream=None):
    """scores -> select -> compact on the GPU; returns a dict of device tensors."""
    C_max = cfg.C_max if C_max is None else C_max
    pool_kernel = cfg.pool_kernel if pool_kernel is None else pool_kernel
    L = inp["q_obs"].shape[0]
    shape = shape_of(cfg, kv_head_stride=inp["kv_head_stride"], n_layers=L)
    ws = workspace(shape, C_max)
    dev = inp["q_obs"].device
    n_pre = cfg.n_in - cfg.n_window
    n_keep = skv.speckv_n_keep(shape, C_max)
    scores = torch.full((L, cfg.n_kv_heads, n_pre), float("nan"), dtype=torch.float32, device=dev)
    pooled = torch.full_like(scores, float("nan"))
    kept = torch.full((L, cfg.n_kv_heads, n_keep), -1, dtype=torch.int32, device=dev)
    skv.speckv_scores(shape, inp["q_obs"], inp["k_buf"], scores, ws, stream)
    skv.speckv_select(shape, scores, C_max, pool, pool_kernel, kept, pooled, ws, stream)
    out = {"scores": scores, "pooled": pooled, "kept": kept, "n_keep": n_keep, "shape": shape, "ws": ws}
    if in_place:
        skv.speckv_compact(shape, inp["k_buf"], inp["v_buf"], kept, n_keep, inp["k_buf"], inp["v_buf"], ws, stream)
        d = cfg.head_dim
        out["k_c"] = inp["k_buf"][:, :, :n_keep * d].unflatten(2, (n_keep, d))
        out["v_c"] = inp["v_buf"][:, :, :n_keep * d].unflatten(2, (n_keep, d))
    else:
        k_c = torch.empty((L, cfg.n_kv_heads, n_keep, cfg.head_dim), dtype=inp["k_buf"].dtype, device=dev)
        v_c = torch.empty_like(k_c)
        skv.speckv_compact(shape, inp["k_buf"], inp["v_buf"], kept, n_keep, k_c, v_c, ws, stream)
        out["k_c"], out["v_c"] = k_c, v_c
    return out


def assert_scores_close(got, want, G, n_obs, what="scores"):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    tol = SCORE_RTOL * np.abs(want) + 1e-12 * G * n_obs
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first {idx.tolist()}: "
                             f"got {got[tuple(idx[0])]!r} want {want[tuple(idx[0])]!r}; "
                             f"max rel {np.max(err / np.maximum(np.abs(want), 1e-300)):.3e}")


def assert_kept_matches(kept_gpu, pooled_gpu, pooled_oracle, C_max, n_window, what="kept"):
    """Per head: (1) the oracle's rule applied to the GPU's own fp32 pooled
    scores gives exactly the GPU's kept list (same-precision decision); (2)
    against the fp64 oracle, the kept sets differ only at keys whose pooled
    score ties the cut-off within the score tolerance."""
    import oracle
    kept_gpu = np.asarray(kept_gpu)
    n_heads = kept_gpu.shape[0]
    for h in range(n_heads):
        kg = kept_gpu[h]
        exact = oracle.select_kept(np.asarray(pooled_gpu[h], dtype=np.float64), C_max, n_window)
        assert kg.tolist() == exact.tolist(), f"{what}[{h}]: GPU selection differs from the rule on its own scores"
        po = np.asarray(pooled_oracle[h], dtype=np.float64)
        ko = oracle.select_kept(po, C_max, n_window)
        assert len(kg) == len(ko)
        n_top = len(ko) - n_window
        assert kg[n_top:].tolist() == ko[n_top:].tolist()
        if n_top == 0:
            continue
        thr = np.sort(po)[::-1][n_top - 1]
        for j in set(kg[:n_top].tolist()) ^ set(ko[:n_top].tolist()):
            assert abs(po[j] - thr) <= SCORE_RTOL * thr + 1e-30, \
                f"{what}[{h}]: key {j} differs with pooled {po[j]!r} vs cut-off {thr!r}"


def assert_compacted(k_c, v_c, k, v, kept):
    """Bit-exact rows at the GPU's own kept indices."""
    kept = torch.as_tensor(kept, device=k.device).long()
    idx = kept.unsqueeze(-1).expand(*kept.shape, k.shape[-1])
    assert torch.equal(k_c, torch.gather(k, 2, idx)), "compacted K differs from the source rows"
    assert torch.equal(v_c, torch.gather(v, 2, idx)), "compacted V differs from the source rows"


def np64(t):
    return wl.to_numpy_f64(t)


def raw_host(t):
    """Host copy of a tensor's raw elements (bfloat16 as uint16 words, float32 as is), for the oracle pool."""
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def check_every_unit_against_oracle(scores, pooled, kept, q_obs, k, cfg, per_query_head=False, aggregation="sum",
                                    layer_ids=None, label=""):
    """Compares EVERY (layer, head) unit of a GPU launch with the fp64 oracle,
    the oracle spread over a pool of single-threaded worker processes.

    scores, pooled, kept: host arrays [L, H, ...] from the GPU; q_obs, k:
    the inputs (device or host tensors) [L, Hq, n_obs, d] and [L, Hkv, n_in, d].
    Per unit: scores within the tolerance, the selection rule exact on the
    GPU's own pooled scores and equal to the oracle's up to ties within the
    tolerance.  layer_ids names the layers in messages (default 0 ..)."""
    import time
    import oracle
    from oracle.pool import OraclePool, worker_count
    L, H = kept.shape[:2]
    G = cfg.G
    rows = 1 if per_query_head else G
    layer_ids = list(range(L)) if layer_ids is None else list(layer_ids)
    q_raw, k_raw = raw_host(q_obs), raw_host(k)
    scale = oracle.default_scale(cfg.head_dim)

    def tasks():
        for u in range(L * H):
            layer, h = divmod(u, H)
            q = q_raw[layer, h:h + 1] if per_query_head else q_raw[layer, h * G:(h + 1) * G]
            kvh = h // G if per_query_head else h
            yield dict(uid=u, q=q, k=k_raw[layer, kvh], n_pre=cfg.n_pre, scale=scale, aggregation=aggregation)

    n = worker_count()
    print(f"[oracle] {label}: {L * H} units on {n} worker processes", flush=True)
    t0, done = time.perf_counter(), 0
    with OraclePool(n) as pool:
        for u, want, _ in pool.imap("speckv", tasks()):
            layer, h = divmod(u, H)
            where = f"{label}[layer {layer_ids[layer]}, head {h}]"
            assert_scores_close(scores[layer, h], want, rows, cfg.n_obs, f"scores{where}")
            assert_kept_matches(kept[layer, h][None], pooled[layer, h][None],
                                oracle.pool1d(want, cfg.pool_kernel, "max")[None], cfg.C_max, cfg.n_window,
                                f"kept{where}")
            done += 1
            if done % 64 == 0 or done == L * H:
                print(f"[oracle] {label}: {done} of {L * H} units match ({time.perf_counter() - t0:.0f} s)",
                      flush=True)
