"""bench.py's host-side pieces on small inputs: the fp64 oracle baselines of
the SpecKV, SpecPC, cascade and decode lines run on a pool of single-threaded
workers (one per core, at most 16) and report positive rates with the worker
count as `cores` and a single-core extrapolation; the step statistics and the
input digests; the vector-unit peaks."""
import dataclasses
import hashlib

import pytest
import torch

import bench
from attention_importance_scoring_amd import workloads as wl
from oracle.pool import worker_count


def test_vector_peaks_from_unit_counts_and_measured_issue_cycles():
    # 256 CUs x 4 SIMDs x 64 lanes at 2.4 GHz over the measured wave64 issue cycles
    assert bench.PEAK_EXP_TPS == pytest.approx(256 * 4 * 64 / 9.04 * 2.4e9 / 1e12)
    assert bench.PEAK_ELEM_TPS == pytest.approx(256 * 4 * 64 / (3.05 + 9.04 + 4.49) * 2.4e9 / 1e12)
    assert 9.4 < bench.PEAK_ELEM_TPS < 9.6 and bench.PEAK_MIX_ELEM_TPS < bench.PEAK_ELEM_TPS


def _check_pool_fields(out):
    assert out["kind"] == "oracle" and out["value"] > 0
    assert out["cores"] == worker_count() and "single-threaded" in out["sample"]


def test_speckv_baseline_small():
    cfg = wl.reduced(wl.QWEN32B_64K, n_layers=2, n_in=2048, n_lookahead=16)
    out = bench.speckv_cpu_baseline(cfg, wl.speckv_inputs(cfg, 3, "cpu"), budget_s=0.2)
    _check_pool_fields(out)
    ex = out["single_core_extrapolated"]
    assert ex["units"] == 16 and ex["step_s"] == pytest.approx(ex["unit_s"] * 16, rel=1e-3, abs=2e-3)


def test_specpc_baseline_small_and_with_lookahead():
    for la in (1, 16):
        cfg = wl.reduced(wl.SPECPC_DRAFT_32K, n_layers=4, l_skip=1, n_in=2048, window=128, k_top=200, n_lookahead=la)
        out = bench.specpc_cpu_baseline(cfg, wl.specpc_inputs(cfg, 5, "cpu"))
        _check_pool_fields(out)
        assert out["unit"] == "tokens/s" and "42 causal window maps" in out["sample"]


def test_specpc_pool_equals_the_sequential_oracle():
    import numpy as np
    import oracle
    cfg = wl.reduced(wl.SPECPC_DRAFT_32K, n_layers=3, l_skip=1, n_in=1024, window=64, k_top=100)
    inp = wl.specpc_inputs(cfg, 5, "cpu")
    _, tokens, _, _ = bench._specpc_oracle_pool(cfg, inp, 2)
    want = oracle.specpc_token_scores(wl.to_numpy_f64(inp["q_win"]), wl.to_numpy_f64(inp["k"]), cfg.l_skip)
    ref, _ = oracle.specpc_select(want, cfg.k_top, "max", cfg.pool_kernel)
    assert np.array_equal(np.asarray(tokens), ref)


def test_cascade_baseline_small():
    base = wl.CASCADES["speckv_pc_cascade_32k"]
    cc = dataclasses.replace(base, draft=wl.reduced(base.draft, n_layers=4, l_skip=1, n_in=2048, window=128,
                                                    k_top=256),
                             target=wl.reduced(base.target, n_layers=1, n_in=2048))
    out = bench.cascade_cpu_baseline(cc, wl.cascade_inputs(cc, 5, "cpu"))
    _check_pool_fields(out)
    assert "256-token prompt" in out["sample"]


def test_decode_baseline_small():
    cfg = wl.reduced(wl.QWEN32B_64K, n_layers=2, n_in=1024, n_lookahead=16, C_max=64)
    out = bench.decode_cpu_baseline(cfg, wl.speckv_inputs(cfg, 3, "cpu"), "compacted", budget_s=0.2)
    _check_pool_fields(out)


def test_step_stats_and_input_digests():
    st = bench.step_stats([3.0, 1.0, 2.0, 5.0])
    assert st == {"ms_per_step_median": 2.5, "ms_per_step_min": 1.0}
    t = torch.arange(24, dtype=torch.float32).reshape(2, 3, 4).to(torch.bfloat16)
    combined, per_layer = bench.input_digests({"x": t})
    want0 = hashlib.sha256(t[0].contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()
    assert per_layer["x"][0] == want0 and len(per_layer["x"]) == 2
    assert combined["x"] == hashlib.sha256("".join(per_layer["x"]).encode()).hexdigest()
