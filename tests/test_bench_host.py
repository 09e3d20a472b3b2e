"""bench.py's host-side pieces on small inputs: the fp64 oracle baselines of
the SpecKV, SpecPC and cascade lines run and report positive rates, and the
derived exp peak is 256 CUs x 32 per clock x 2.4 GHz."""
import dataclasses

import pytest

import bench
from attention_importance_scoring_amd import workloads as wl


def test_exp_peak_from_unit_counts():
    assert bench.PEAK_EXP_TPS == pytest.approx(19.6608)


def test_speckv_baseline_small():
    cfg = wl.reduced(wl.QWEN32B_64K, n_layers=1, n_in=2048, n_lookahead=16)
    out = bench.speckv_cpu_baseline(cfg, wl.speckv_inputs(cfg, 3, "cpu"), budget_s=0.2)
    assert out["kind"] == "oracle" and out["value"] > 0 and out["cores"] >= 1


def test_specpc_baseline_small_and_with_lookahead():
    for la in (1, 16):
        cfg = wl.reduced(wl.SPECPC_DRAFT_32K, n_layers=4, l_skip=1, n_in=2048, window=128, k_top=200, n_lookahead=la)
        out = bench.specpc_cpu_baseline(cfg, wl.specpc_inputs(cfg, 5, "cpu"), budget_s=0.2)
        assert out["unit"] == "tokens/s" and out["value"] > 0
        assert "of 3 used layers" in out["sample"]


def test_cascade_baseline_small():
    base = wl.CASCADES["speckv_pc_cascade_32k"]
    cc = dataclasses.replace(base, draft=wl.reduced(base.draft, n_layers=4, l_skip=1, n_in=2048, window=128,
                                                    k_top=256),
                             target=wl.reduced(base.target, n_layers=1, n_in=2048))
    out = bench.cascade_cpu_baseline(cc, wl.cascade_inputs(cc, 5, "cpu"), budget_s=0.4)
    assert out["value"] > 0 and "256-token prompt" in out["sample"]
