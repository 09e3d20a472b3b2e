"""The peak-check program (attention_importance_scoring_amd/peaks/peaks.hip)
runs every test on the GPU and reports positive rates and clocks.  Its full
run gives the measured ceilings beside the datasheet peaks; this runs its
small mode."""
import json
import os
import subprocess

import pytest

from attention_importance_scoring_amd import build

pytestmark = pytest.mark.gpu


def test_peak_checks_small_run():
    print("\n[case] skv_peaks --small", flush=True)
    assert os.path.exists(build.PEAKS_BIN), "peak-check program not built (run build())"
    r = subprocess.run([build.PEAKS_BIN, "--small"], capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, r.stderr
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["small"] is True
    assert out["hbm_read_GBps"] > 0 and out["hbm_copy_GBps"] > 0
    assert all(v > 0 for v in out["mfma_bf16_TFLOPs"]) and all(v > 0 for v in out["exp_T_per_s"])
    assert all(v > 0 for v in out["clock_GHz"]["mfma"])
