"""speckv_select on given scores: pooling and top-C_max selection against the
oracle's pool1d and select_kept (paper notes "Draft-based Approximate
Inference for LLMs", section "Key designs": SpecKV keeps the top C_max pairs
plus the window; section "Loss / training strategy": local pooling).

The scores are inputs here, so max pooling and no pooling are exact in fp32:
the GPU's pooled values equal the oracle's bit for bit and the kept lists must
be identical, ties to the lowest index included.  Mean pooling sums in fp32 on
the GPU: its pooled values are checked to a relative 1e-6 and its kept list
against the oracle's rule applied to the GPU's own pooled values.

The cases reach every selection form: one block per unit with the keys in
registers (unit counts of 128 and more), two stages over segments (fewer
units), the single-block radix select beyond 64K keys per block, max pools of
widths up to 65 in registers and other pools through the pooled buffer, and
score sets whose cut-off is tied (plateaus from max pooling, rounded values,
constants), distinct, signed, or tiny."""
import numpy as np
import pytest
import torch

import attention_importance_scoring_amd as skv
import oracle

pytestmark = pytest.mark.gpu


def _scores(kind, units, n, seed):
    g = np.random.default_rng(seed)
    if kind == "heavy":
        s = np.exp(g.normal(0.0, 2.0, (units, n)))
    elif kind == "rounded":
        s = np.round(g.random((units, n)) * 6.0)
    elif kind == "constant":
        s = np.full((units, n), 0.25)
    elif kind == "signed":
        s = g.normal(0.0, 1.0, (units, n))
        s[:, ::11] = -0.0
        s[:, 5::11] = 0.0
    elif kind == "tiny":
        s = g.random((units, n)) * 1e-38  # subnormal and near-subnormal fp32
    elif kind == "plateaus":
        s = np.exp(g.normal(0.0, 2.0, (units, n)))
        s = oracle.pool1d(s.astype(np.float32).astype(np.float64), 5, "max")
    else:
        raise ValueError(kind)
    return s.astype(np.float32)


def _run(units, n_pre, n_window, C_max, pool, pool_kernel, kind, seed=0, pooled_out=True):
    print(f"\n[case] select units={units} n_pre={n_pre} window={n_window} C_max={C_max} pool={pool}/{pool_kernel} "
          f"{kind} pooled_out={pooled_out}", flush=True)
    shape = skv.make_shape(1, units, units, 64, n_pre + n_window, n_window, 0, skv.SKV_F32)
    sc_host = _scores(kind, units, n_pre, seed)
    sc = torch.from_numpy(sc_host).cuda()
    n_keep = skv.speckv_n_keep(shape, C_max)
    ws = torch.empty(max(1, skv.speckv_workspace_bytes(shape, C_max)), dtype=torch.uint8, device="cuda")
    kept = torch.full((1, units, n_keep), -1, dtype=torch.int32, device="cuda")
    pooled = torch.full((1, units, n_pre), -7.0, device="cuda") if pooled_out else None
    pool_id = {"max": skv.SKV_POOL_MAX, "avg": skv.SKV_POOL_AVG, "none": skv.SKV_POOL_NONE}[pool]
    skv.speckv_select(shape, sc.view(1, units, n_pre), C_max, pool_id, pool_kernel, kept, pooled, ws)
    torch.cuda.synchronize()
    kept = kept.cpu().numpy()[0]
    want_pool = oracle.pool1d(sc_host.astype(np.float64), pool_kernel, pool)
    if pooled_out:
        got_pool = pooled.cpu().numpy()[0].astype(np.float64)
        if pool == "avg":
            np.testing.assert_allclose(got_pool, want_pool, rtol=1e-6, atol=1e-45)
        else:
            assert np.array_equal(got_pool, want_pool), "pooled values differ"
    for u in range(units):
        ref_pool = got_pool[u] if (pool == "avg" and pooled_out) else want_pool[u]
        if pool == "avg" and not pooled_out:
            continue  # checked with the pooled output in the other cases
        want = oracle.select_kept(ref_pool, C_max, n_window)
        assert kept[u].tolist() == want.tolist(), f"unit {u}: kept list differs"


@pytest.mark.parametrize("kind", ["heavy", "plateaus", "rounded", "constant", "signed", "tiny"])
def test_registers_64k_keys_per_block(kind):
    # 128 units of 65504 keys: one 1024-thread block per unit, 64 keys per lane
    _run(128, 65504, 32, 256, "max", 7, kind)


@pytest.mark.parametrize("pool,k", [("max", 7), ("none", 1), ("max", 1), ("max", 9), ("avg", 5), ("avg", 1)])
def test_pool_forms(pool, k):
    _run(130, 20000, 16, 300, pool, k, "heavy", seed=3)


@pytest.mark.parametrize("k", [3, 5, 13, 15, 33, 43, 63, 65, 67])
def test_max_pool_widths(k):
    # widths up to 65 pool in registers (doubling windows), 67 through the pooled buffer;
    # 64 keys per lane (direct) and a few per lane (two stages)
    _run(128, 65504, 8, 256, "max", k, "heavy", seed=k)
    _run(2, 30000, 3, 700, "max", k, "plateaus", seed=k + 1)


@pytest.mark.parametrize("n_pre", [100, 5000, 10000], ids=["e4", "e8", "e16"])
@pytest.mark.parametrize("k", [5, 43])
def test_max_pool_widths_fewer_keys_per_lane(n_pre, k):
    # the register pool of a run-time radius at 1, 5 and 10 keys per lane (one block per unit)
    _run(130, n_pre, 3, 64, "max", k, "heavy", seed=n_pre + k)


def test_two_stage_long_segments_other_width():
    # segments of 33334 keys (64 per lane) with a width-15 max pool
    _run(2, 200000, 0, 6000, "max", 15, "heavy", seed=13)


@pytest.mark.parametrize("C_max", [1, 2, 99, 100, 150])
def test_short_units_and_extreme_counts(C_max):
    # 100 keys per unit (every lane but a few is padding); C_max = 1, n_pre - 1, n_pre, above
    _run(130, 100, 4, C_max, "max", 7, "rounded", seed=C_max)


@pytest.mark.parametrize("kind", ["heavy", "plateaus", "rounded"])
def test_two_stage_segments(kind):
    # few units: segments keep their own top C_max, a second block merges them
    _run(2, 32768, 0, 2048, "max", 7, kind, seed=5)
    _run(3, 5001, 7, 64, "max", 7, kind, seed=6)


def test_two_stage_other_pool_widths():
    _run(2, 40000, 3, 500, "max", 15, "heavy", seed=8)
    _run(2, 40000, 3, 500, "none", 1, "rounded", seed=9)


def test_radix_select_beyond_register_capacity():
    # one unit of 300000 keys with a count too large for the two-stage form
    _run(1, 300000, 5, 60000, "max", 7, "heavy", seed=10)


def test_without_pooled_output():
    _run(128, 65504, 32, 256, "max", 7, "plateaus", seed=11, pooled_out=False)
    _run(2, 32768, 0, 2048, "none", 1, "heavy", seed=12, pooled_out=False)
