"""Seeded synthetic inputs for the SpecKV / SpecPC scoring path.

This module draws random inputs only; it holds none of the method's
arithmetic, and both the HIP path and the fp64 oracle consume the very same
bytes it produces.  Generation runs on any torch device (on the GPU for the
large workloads, which are then copied to the host for the oracle).

Workload shapes follow the models the paper notes ("Draft-based Approximate
Inference for LLMs", sections "Background", "Main experiments" with Table 1,
and "Limitations") name: a Llama-3.1-8B-shaped target (32 layers, 32 query /
8 KV heads, head_dim 128), a Qwen2.5-32B-shaped target (64 layers, 40 / 8
heads, head_dim 128) and a Qwen2.5-0.5B-class draft (24 layers, 14 / 2
heads, head_dim 64).  The pages' LongBench / RULER workloads are replaced by the
synthetic key distributions below:

* heavy hitters: a key k_j = beta * sqrt(d) * u + noise, with u the unit mean
  direction of the observation queries of its KV-head group, at random prefix
  positions plus an attention sink at position 0;
* "lowrank8": keys N(0, I) plus a per-head random rank-8 component U_h z_j,
  U_h ~ N(0, 1/8), z_j ~ N(0, I_8);
* "mixture": 90% N(0, I) keys, 10% (random positions) drawn as c_m + 0.1 N(0, I)
  around 64 random centroids c_m ~ N(0, I) per head.

The SpecKV-PC cascade (section "Key designs", SpecKV-PC) pairs the draft
workload with a Qwen2.5-32B-shaped target cache over the same 32K prompt;
SpecPC keeps 2048 tokens and SpecKV then keeps 256 pairs per KV head.

Everything is drawn in fp32 and rounded once to the storage dtype
(round-to-nearest-even for bf16).
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class SpecKVConfig:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str            # "f32" | "bf16"
    n_in: int
    n_window: int
    n_lookahead: int
    C_max: int
    pool_kernel: int
    keys: str             # "normal" | "lowrank8" | "mixture"
    heavy_hitters: str    # "none" | "fixed8" | "one_percent"
    beta: float
    in_place: bool = False

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_obs(self) -> int:
        return self.n_window + self.n_lookahead

    @property
    def n_pre(self) -> int:
        return self.n_in - self.n_window

    @property
    def n_keep(self) -> int:
        return min(self.C_max, self.n_pre) + self.n_window

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def keys_per_call(self) -> int:
        return self.n_layers * self.n_kv_heads * self.n_in


@dataclasses.dataclass(frozen=True)
class SpecPCConfig:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    n_in: int
    window: int           # W window queries (the last W input positions)
    n_lookahead: int
    l_skip: int
    k_top: int
    pool_kernel: int
    beta: float

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_keys(self) -> int:
        """Positions of the draft's query and key axes: n_in + n_lookahead - 1 (n_in when n_lookahead <= 1)."""
        return self.n_in + max(self.n_lookahead, 1) - 1

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


TINY_FP32_2K = SpecKVConfig("tiny_fp32_2k", 1, 4, 1, 64, "f32", 2048, 32, 16, 256, 7, "normal", "fixed8", 3.0)
LLAMA8B_16K = SpecKVConfig("llama8b_shape_16k", 32, 32, 8, 128, "bf16", 16384, 32, 64, 1024, 7, "normal",
                           "one_percent", 2.5)
QWEN32B_64K = SpecKVConfig("qwen32b_shape_64k", 64, 40, 8, 128, "bf16", 65536, 32, 128, 256, 7, "lowrank8",
                           "one_percent", 2.5)
LLAMA8B_128K_INPLACE = SpecKVConfig("llama8b_shape_128k_inplace", 32, 32, 8, 128, "bf16", 131072, 64, 256, 2048, 7,
                                    "mixture", "none", 0.0, in_place=True)
SPECPC_DRAFT_32K = SpecPCConfig("specpc_draft_32k", 24, 14, 2, 64, "bf16", 32768, 512, 1, 4, 2048, 7, 2.5)

WORKLOADS = {c.name: c for c in (TINY_FP32_2K, LLAMA8B_16K, QWEN32B_64K, LLAMA8B_128K_INPLACE, SPECPC_DRAFT_32K)}


@dataclasses.dataclass(frozen=True)
class CascadeConfig:
    """SpecKV-PC: SpecPC keeps draft.k_top of the draft.n_in prompt tokens,
    then SpecKV runs on the target's cache over those tokens.  `target`
    describes the target cache over the FULL prompt (n_in = draft.n_in); its
    rows at the kept tokens stand in for the target's prefill of the
    compressed prompt.  `stage2` is the SpecKV shape over the kept tokens."""
    name: str
    draft: SpecPCConfig
    target: SpecKVConfig

    @property
    def stage2(self) -> SpecKVConfig:
        return dataclasses.replace(self.target, name=self.name + "_stage2", n_in=self.draft.k_top)


CASCADES = {
    "speckv_pc_cascade_32k": CascadeConfig(
        "speckv_pc_cascade_32k", SPECPC_DRAFT_32K,
        SpecKVConfig("qwen32b_shape_32k_target", 64, 40, 8, 128, "bf16", 32768, 32, 128, 256, 7, "lowrank8",
                     "one_percent", 2.5)),
}

_TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "hh": 4, "lowrank": 5, "mix": 6}


def _gen(seed: int, layer: int, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + layer * 10_007 + _TENSOR_IDS[tensor] * 101) % (2**63 - 1))
    return g


def _randn(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _unit_mean_direction(q_rows: torch.Tensor) -> torch.Tensor:
    """q_rows: [Hkv, rows, d] -> unit mean direction per KV head [Hkv, d]."""
    u = q_rows.mean(dim=1)
    return u / u.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def _heavy_hitter_positions(kind: str, n_in: int, n_pre: int, g, device) -> torch.Tensor:
    if kind == "fixed8":
        # eight positions on a stride-7 grid so that their pooling plateaus are disjoint
        slots = torch.randperm(n_pre // 7 - 1, generator=g, device=device)[:8]
        return 7 * slots + 4
    if kind == "one_percent":
        n_hh = n_in // 100
        return torch.randperm(n_pre - 1, generator=g, device=device)[:n_hh] + 1
    raise ValueError(kind)


def speckv_layer(cfg: SpecKVConfig, layer: int, seed: int, device="cpu", planted=None):
    """One layer of inputs: q_obs [Hq, n_obs, d], k [Hkv, n_in, d], v [Hkv, n_in, d].

    planted: None, or a list to which the positions of the planted keys
    (heavy hitters and the sink at 0) of each KV head are appended (the
    positions themselves, not anything computed from them)."""
    d, Hq, Hkv, G = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.G
    q = _randn((Hq, cfg.n_obs, d), _gen(seed, layer, "q", device), device)
    k = _randn((Hkv, cfg.n_in, d), _gen(seed, layer, "k", device), device)
    if cfg.keys == "lowrank8":
        gl = _gen(seed, layer, "lowrank", device)
        U = _randn((Hkv, d, 8), gl, device) / math.sqrt(8.0)
        z = _randn((Hkv, cfg.n_in, 8), gl, device)
        k += torch.bmm(z, U.transpose(1, 2).contiguous())
    elif cfg.keys == "mixture":
        gm = _gen(seed, layer, "mix", device)
        n_cl = cfg.n_in // 10
        for h in range(Hkv):
            pos = torch.randperm(cfg.n_in, generator=gm, device=device)[:n_cl]
            cent = _randn((64, d), gm, device)
            which = torch.randint(0, 64, (n_cl,), generator=gm, device=device)
            k[h, pos] = cent[which] + 0.1 * _randn((n_cl, d), gm, device)
    if cfg.heavy_hitters != "none":
        gh = _gen(seed, layer, "hh", device)
        q_rounded = q.to(cfg.torch_dtype).float()
        u = _unit_mean_direction(q_rounded.reshape(Hkv, G * cfg.n_obs, d))
        for h in range(Hkv):
            pos = _heavy_hitter_positions(cfg.heavy_hitters, cfg.n_in, cfg.n_pre, gh, device)
            pos = torch.cat([torch.zeros(1, dtype=pos.dtype, device=device), pos])
            k[h, pos] = cfg.beta * math.sqrt(d) * u[h] + _randn((pos.numel(), d), gh, device)
            if planted is not None:
                planted.append(pos.cpu())
    v = _randn((Hkv, cfg.n_in, d), _gen(seed, layer, "v", device), device)
    dt = cfg.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def speckv_inputs(cfg: SpecKVConfig, seed: int, device="cpu", layers=None, kv_head_stride=None):
    """Stacked inputs for the given layers (default: all).

    Returns dict with q_obs [L, Hq, n_obs, d], k and v as [L, Hkv, n_in, d]
    views (when kv_head_stride is given, k and v are views of a larger
    buffer whose head slabs are kv_head_stride elements apart), and
    "planted": per layer, per KV head, the planted key positions (empty lists
    when the workload plants none).
    """
    layers = list(range(cfg.n_layers)) if layers is None else list(layers)
    L, d = len(layers), cfg.head_dim
    dt = cfg.torch_dtype
    stride = cfg.n_in * d if kv_head_stride is None else int(kv_head_stride)
    assert stride >= cfg.n_in * d
    q_obs = torch.empty((L, cfg.n_q_heads, cfg.n_obs, d), dtype=dt, device=device)
    kbuf = torch.empty((L, cfg.n_kv_heads, stride), dtype=dt, device=device)
    vbuf = torch.empty((L, cfg.n_kv_heads, stride), dtype=dt, device=device)
    planted = []
    for i, layer in enumerate(layers):
        pl = []
        q, k, v = speckv_layer(cfg, layer, seed, device, planted=pl)
        planted.append(pl)
        q_obs[i] = q
        kbuf[i, :, :cfg.n_in * d] = k.reshape(cfg.n_kv_heads, -1)
        vbuf[i, :, :cfg.n_in * d] = v.reshape(cfg.n_kv_heads, -1)
    k_view = kbuf[:, :, :cfg.n_in * d].unflatten(2, (cfg.n_in, d))
    v_view = vbuf[:, :, :cfg.n_in * d].unflatten(2, (cfg.n_in, d))
    return {"q_obs": q_obs, "k": k_view, "v": v_view, "k_buf": kbuf, "v_buf": vbuf, "kv_head_stride": stride,
            "planted": planted}


def specpc_layer(cfg: SpecPCConfig, layer: int, seed: int, device="cpu"):
    """One draft layer: q_win [Hq, W, d] (window queries), k [Hkv, n_keys, d]
    (n_keys = n_in + n_lookahead - 1: the input tokens, then the draft tokens
    the window's last rows are)."""
    d, Hq, Hkv, G, W = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.G, cfg.window
    q = _randn((Hq, W, d), _gen(seed, layer, "q", device), device)
    k = _randn((Hkv, cfg.n_keys, d), _gen(seed, layer, "k", device), device)
    gh = _gen(seed, layer, "hh", device)
    q_rounded = q.to(cfg.torch_dtype).float()
    u = _unit_mean_direction(q_rounded.reshape(Hkv, G * W, d))
    n_pre = min(cfg.n_keys - W, cfg.n_in)  # planted keys are input tokens before the window
    n_hh = min(cfg.n_in // 100, max(n_pre - 1, 0))
    for h in range(Hkv):
        pos = torch.randperm(max(n_pre - 1, 0), generator=gh, device=device)[:n_hh] + 1
        pos = torch.cat([torch.zeros(1, dtype=pos.dtype, device=device), pos])
        k[h, pos] = cfg.beta * math.sqrt(d) * u[h] + _randn((pos.numel(), d), gh, device)
    dt = cfg.torch_dtype
    return q.to(dt), k.to(dt)


def specpc_inputs(cfg: SpecPCConfig, seed: int, device="cpu"):
    """q_win [L, Hq, W, d] and k [L, Hkv, n_keys, d] for all layers (skipped ones included)."""
    L, d = cfg.n_layers, cfg.head_dim
    dt = cfg.torch_dtype
    q_win = torch.empty((L, cfg.n_q_heads, cfg.window, d), dtype=dt, device=device)
    k = torch.empty((L, cfg.n_kv_heads, cfg.n_keys, d), dtype=dt, device=device)
    for layer in range(L):
        q_win[layer], k[layer] = specpc_layer(cfg, layer, seed, device)
    return {"q_win": q_win, "k": k}


def cascade_inputs(cc: CascadeConfig, seed: int, device="cpu", target_layers=None):
    """Draft inputs (seed) and the target's full-prompt cache and observation
    queries (seed + 1): {"draft": specpc_inputs(...), "target": speckv_inputs(...)}.
    The draft's and the target's planted keys are drawn independently."""
    return {"draft": specpc_inputs(cc.draft, seed, device),
            "target": speckv_inputs(cc.target, seed + 1, device, layers=target_layers)}


def reduced(cfg, **changes):
    """A copy of a config with some fields changed (smaller parity cases)."""
    return dataclasses.replace(cfg, **changes)


def to_numpy_f64(t: torch.Tensor):
    """Exact host copy as float64 (bf16 and fp32 values are exact in float64)."""
    return t.detach().to("cpu", torch.float32).double().numpy()
