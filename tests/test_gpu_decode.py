"""GPU parity of decode attention over a (compacted) KV cache through the C
ABI, against the fp64 oracle (oracle/decode.py).

Tolerance, per output component: |gpu - oracle| <= 2e-4 * sum_j P_j |v_j|
(oracle.error_scale).  The kernel's bf16 x bf16 products are exact (fp32
products round once) and accumulate in fp32 over the head dim (a logit
error of at most d * 2^-24 * sum |q_c k_c| * scale, under 6e-5 for the
N(0, 1) inputs here), exp2 is correct to about one ulp, P enters the P V
product as two bf16 terms (relative error at most 2^-18; exact for fp32
caches) and the sums over rows run in fp32: each
probability is off by well under 1e-4 relative, which moves an output
component by at most twice that in units of sum_j P_j |v_j|.
"""
import numpy as np
import pytest
import torch

import attention_importance_scoring_amd as skv
import oracle
from attention_importance_scoring_amd import workloads as wl

from gpu_helpers import np64, run_speckv

pytestmark = pytest.mark.gpu

DECODE_TOL = 2e-4


def _cache(L, H, n_alloc, d, seed, device="cuda", scale_k=1.0, stride=None, dtype=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(seed)
    stride = n_alloc * d if stride is None else stride
    kb = torch.randn((L, H, stride), generator=g).mul_(scale_k).to(dtype)
    vb = torch.randn((L, H, stride), generator=g).to(dtype)
    return kb.to(device), vb.to(device)


def _decode(shape, n_rows, q, kb, vb, L, Hq, d):
    ws_n = skv.speckv_decode_workspace_bytes(shape, n_rows)
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device="cuda") if ws_n else None
    out = torch.full((L, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    skv.speckv_decode_attention(shape, n_rows, q, kb, vb, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _check(got, q, k, v, n_rows, what):
    want = oracle.decode_attention(q, k, v, n_rows)
    es = oracle.error_scale(q, k, v, n_rows)
    err = np.abs(got - want)
    bad = err > DECODE_TOL * es
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; max err/scale "
                           f"{np.max(err / es):.3e} at {np.unravel_index(np.argmax(err / es), err.shape)}")
    return float(np.max(err / es))


@pytest.mark.parametrize("L,Hq,Hkv,d,n_alloc,n_rows,pqh,dt", [
    (2, 8, 2, 128, 300, 300, 0, "bf16"),      # ragged single chunk, G 4
    (1, 40, 8, 128, 288, 288, 0, "bf16"),     # the compacted 64K Qwen-shaped cache: G 5, 288 rows
    (2, 14, 2, 64, 2049, 2049, 0, "bf16"),    # d 64, G 7, five chunks with a one-row tail
    (1, 8, 8, 128, 40, 40, 0, "bf16"),        # G 1, two tiles: two of four waves idle
    (2, 8, 2, 128, 1000, 288, 0, "bf16"),     # rows attended < rows allocated (in-place compacted layout)
    (1, 16, 1, 64, 600, 517, 0, "bf16"),      # G 16 (the MFMA width), a 5-row second chunk
    (2, 8, 2, 128, 200, 200, 1, "bf16"),      # one cache per query head
    (2, 8, 2, 128, 300, 300, 0, "f32"),       # fp32: ragged, two 256-key chunks
    (1, 4, 1, 64, 288, 288, 0, "f32"),        # fp32 d 64: the compacted tiny fp32 cache (G 4)
    (2, 14, 2, 64, 2049, 2049, 0, "f32"),     # fp32 d 64, G 7, nine chunks with a one-row tail
    (1, 16, 1, 128, 600, 517, 0, "f32"),      # fp32 G 16, rows attended < allocated
    (2, 8, 2, 128, 200, 200, 1, "f32"),       # fp32, one cache per query head
])
def test_decode_small(L, Hq, Hkv, d, n_alloc, n_rows, pqh, dt):
    H = Hq if pqh else Hkv
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    print(f"\n[case] {dt} L={L} Hq={Hq} H={H} d={d} rows {n_rows} of {n_alloc}", flush=True)
    kb, vb = _cache(L, H, n_alloc, d, seed=n_rows + d, dtype=tdt)
    q = torch.randn((L, Hq, d), generator=torch.Generator().manual_seed(3)).to(tdt).cuda()
    shape = skv.make_shape(L, Hq, Hkv, d, n_alloc, 0, 0, skv.SKV_F32 if dt == "f32" else skv.SKV_BF16,
                           per_query_head=pqh)
    got = _decode(shape, n_rows, q, kb, vb, L, Hq, d)
    k = np64(kb.view(L, H, n_alloc, d))
    v = np64(vb.view(L, H, n_alloc, d))
    _check(got, np64(q), k, v, n_rows, "decode")


def test_single_row_is_exact_and_padded_stride():
    L, Hq, Hkv, d, n_alloc = 1, 10, 2, 128, 7
    stride = n_alloc * d + 64  # padded head slabs
    kb, vb = _cache(L, Hkv, n_alloc, d, seed=5, stride=stride)
    q = torch.randn((L, Hq, d), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16).cuda()
    shape = skv.make_shape(L, Hq, Hkv, d, n_alloc, 0, 0, skv.SKV_BF16, kv_head_stride=stride)
    got = _decode(shape, 1, q, kb, vb, L, Hq, d)
    v0 = np64(vb[:, :, :d])
    for hq in range(Hq):
        np.testing.assert_array_equal(got[0, hq], v0[0, hq // 5])
    got = _decode(shape, n_alloc, q, kb, vb, L, Hq, d)
    k = np64(kb[:, :, :n_alloc * d].reshape(L, Hkv, n_alloc, d))
    v = np64(vb[:, :, :n_alloc * d].reshape(L, Hkv, n_alloc, d))
    _check(got, np64(q), k, v, n_alloc, "padded stride")


def test_peaked_and_flat_logits():
    # large logits (one key far above the rest) and all-equal keys
    L, Hq, Hkv, d, n = 1, 4, 1, 128, 700
    kb, vb = _cache(L, Hkv, n, d, seed=7, scale_k=6.0)
    q = (6.0 * torch.randn((L, Hq, d), generator=torch.Generator().manual_seed(8))).to(torch.bfloat16).cuda()
    shape = skv.make_shape(L, Hq, Hkv, d, n, 0, 0, skv.SKV_BF16)
    got = _decode(shape, n, q, kb, vb, L, Hq, d)
    _check(got, np64(q), np64(kb.view(L, Hkv, n, d)), np64(vb.view(L, Hkv, n, d)), n, "peaked")
    kb.view(L, Hkv, n, d)[:] = kb.view(L, Hkv, n, d)[:, :, :1]
    got = _decode(shape, n, q, kb, vb, L, Hq, d)
    mean = np64(vb.view(L, Hkv, n, d)).mean(axis=2)
    np.testing.assert_allclose(got[0], np.broadcast_to(mean[0, 0], (Hq, d)), rtol=0, atol=1e-5)


def test_decode_over_the_compacted_cache_of_the_speckv_path():
    # scores -> select -> compact on the GPU, then decode over the compacted cache:
    # equals attention over the GPU's kept rows of the full cache
    cfg = wl.reduced(wl.LLAMA8B_16K, n_layers=2, n_in=3000, C_max=100)
    print(f"\n[case] {cfg.name} reduced: n_in {cfg.n_in}, C_max {cfg.C_max}", flush=True)
    inp = wl.speckv_inputs(cfg, 12, "cuda")
    res = run_speckv(cfg, inp)
    n_keep = res["n_keep"]
    L, Hq, Hkv, d = cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = torch.randn((L, Hq, d), generator=torch.Generator().manual_seed(13)).to(torch.bfloat16).cuda()
    shape = skv.make_shape(L, Hq, Hkv, d, n_keep, 0, 0, skv.SKV_BF16)
    got = _decode(shape, n_keep, q, res["k_c"], res["v_c"], L, Hq, d)
    kept = res["kept"].cpu().numpy()
    k_full, v_full = np64(inp["k"]), np64(inp["v"])
    kc = np.stack([[k_full[layer, h][kept[layer, h]] for h in range(Hkv)] for layer in range(L)])
    vc = np.stack([[v_full[layer, h][kept[layer, h]] for h in range(Hkv)] for layer in range(L)])
    _check(got, np64(q), kc, vc, n_keep, "decode after compaction")


@pytest.mark.parametrize("n_rows", [288, 8292, 65536])
def test_qwen32b_shape_full_layers_sampled(n_rows):
    # the bench launch: all 64 layers' caches in one call (288 rows: the compacted
    # 64K cache; 65536: the full cache, 16 sub-chunks per block; 8292: two sub-chunks
    # per block and a last block with one partial sub-chunk), sampled heads against the oracle
    L, Hq, Hkv, d = 64, 40, 8, 128
    print(f"\n[case] 64 layers x 8 KV heads, {n_rows} rows, one call", flush=True)
    g = torch.Generator(device="cuda").manual_seed(n_rows)
    kb = torch.randn((L, Hkv, n_rows * d), generator=g, device="cuda").to(torch.bfloat16)
    vb = torch.randn((L, Hkv, n_rows * d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((L, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    shape = skv.make_shape(L, Hq, Hkv, d, n_rows, 0, 0, skv.SKV_BF16)
    got = _decode(shape, n_rows, q, kb, vb, L, Hq, d)
    assert np.isfinite(got).all()
    for layer, h in [(0, 0), (33, 5), (63, 7)]:
        k = np64(kb[layer:layer + 1, h:h + 1].view(1, 1, n_rows, d))
        v = np64(vb[layer:layer + 1, h:h + 1].view(1, 1, n_rows, d))
        _check(got[layer:layer + 1, h * 5:(h + 1) * 5], np64(q[layer:layer + 1, h * 5:(h + 1) * 5]), k, v, n_rows,
               f"layer {layer} head {h}")


@pytest.mark.parametrize("direction,dt", [("rising", "bf16"), ("falling", "bf16"), ("rising", "f32")])
def test_running_maximum_across_sub_chunks(direction, dt):
    # logits that rise (or fall) along the cache: with many heads each block walks
    # several sub-chunks and its running maximum changes in every one of them
    L, Hq, Hkv, d, n = 64, 16, 8, 64, 9000
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    print(f"\n[case] {direction} logits {dt}, {L * Hkv} heads x {n} rows", flush=True)
    g = torch.Generator(device="cuda").manual_seed(21)
    u = torch.randn(d, generator=g, device="cuda")
    u = u / u.norm()
    ramp = torch.linspace(0.0, 1.0, n, device="cuda")
    if direction == "falling":
        ramp = ramp.flip(0)
    k = 40.0 * ramp[None, None, :, None] * u + 0.5 * torch.randn((L, Hkv, n, d), generator=g, device="cuda")
    kb = k.to(tdt).reshape(L, Hkv, n * d)
    vb = torch.randn((L, Hkv, n * d), generator=g, device="cuda").to(tdt)
    q = (u[None, None, :] + 0.1 * torch.randn((L, Hq, d), generator=g, device="cuda")).to(tdt)
    shape = skv.make_shape(L, Hq, Hkv, d, n, 0, 0, skv.SKV_F32 if dt == "f32" else skv.SKV_BF16)
    got = _decode(shape, n, q, kb, vb, L, Hq, d)
    for layer, h in [(0, 0), (40, 3), (63, 7)]:
        kk = np64(kb[layer:layer + 1, h:h + 1].view(1, 1, n, d))
        vv = np64(vb[layer:layer + 1, h:h + 1].view(1, 1, n, d))
        _check(got[layer:layer + 1, 2 * h:2 * h + 2], np64(q[layer:layer + 1, 2 * h:2 * h + 2]), kk, vv, n,
               f"{direction} layer {layer} head {h}")
