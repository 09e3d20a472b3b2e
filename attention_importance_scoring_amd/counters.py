"""Summaries of rocprofv3 output for the scoring library's kernels.

Two modes, both reading the CSV files rocprofv3 writes with
``-d DIR -o run --output-format csv``:

* ``--stats DIR``: the ``--kernel-trace --stats`` table (calls, total and
  average duration per kernel) as text.
* ``--fetch DIR --write DIR``: HBM traffic per launch from one
  ``--pmc FETCH_SIZE`` run and one ``--pmc WRITE_SIZE`` run of the same
  command.  Both counters are in KiB per dispatch.  Each is scaled by the
  factor that makes it read exactly right on a plain streaming kernel of
  known size (``bench.py --calib-copy-mib M`` runs ``torch.neg`` over M MiB
  of fp32: M MiB read, M MiB written), and the result is written as JSON
  for ``bench.py`` together with a hash of the kernel sources, so that a
  later change of the kernels voids it.

    python -m attention_importance_scoring_amd.counters --stats out/trace --title "..." --command "..."
    python -m attention_importance_scoring_amd.counters --fetch out/pmc_fetch --write out/pmc_write \\
        --calib-mib 1024 --workload qwen32b_shape_64k --command "..." \\
        --out profiles/speckv_kernels_qwen32b_shape_64k_traffic.json
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ["attention_importance_scoring_amd/csrc/" + f for f in
                  ("common.hpp", "kernels.hpp", "score.hip", "select.hip", "specpc.hip", "decode.hip", "capi.hip")]
CALIB_PATTERN = "neg_kernel"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(kernel_name: str) -> str:
    """'void skv::score_pass1_kernel<skv::bf16_t, 128>(skv::ScoreArgs)' -> 'score_pass1_kernel<bf16_t, 128>'
    (kernels in an anonymous namespace inside skv included)."""
    kernel_name = kernel_name.replace("(anonymous namespace)::", "")
    m = re.search(r"skv::(\w+)(<[^()]*>)?", kernel_name)
    if m:
        return m.group(1) + (m.group(2) or "").replace("skv::", "")
    if CALIB_PATTERN in kernel_name:
        return "calibration:torch.neg"
    return kernel_name.split("(")[0][-60:]


def _csv(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def stats_table(d: str) -> list[dict]:
    rows = []
    with open(_csv(d, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "total_ms": float(r["TotalDurationNs"]) * 1e-6, "avg_us": float(r["AverageNs"]) * 1e-3,
                         "pct": float(r["Percentage"])})
    return rows


def per_dispatch(d: str, counter: str, reduce: str = "sum") -> dict[str, list[float]]:
    """Counter value per dispatch (summed, or the maximum, over the dimensions rocprofv3
    reports), grouped by kernel."""
    by_dispatch = {}
    name_of = {}
    with open(_csv(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            v = float(r["Counter_Value"])
            if key not in by_dispatch:
                by_dispatch[key] = v
            else:
                by_dispatch[key] = max(by_dispatch[key], v) if reduce == "max" else by_dispatch[key] + v
            name_of[key] = short_name(r["Kernel_Name"])
    out = collections.defaultdict(list)
    for key in sorted(by_dispatch):
        out[name_of[key]].append(by_dispatch[key])
    return out


def traffic(fetch_dir: str, write_dir: str, calib_mib: int) -> dict:
    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    calib = "calibration:torch.neg"
    known_kib = calib_mib * 1024.0
    if calib not in fetch or calib not in write:
        raise SystemExit("calibration kernel not found: run bench.py with --calib-copy-mib")
    # the largest dispatches of the calibration kernel are the M MiB runs
    f_cal = max(fetch[calib])
    w_cal = max(write[calib])
    f_scale, w_scale = known_kib / f_cal, known_kib / w_cal
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        if not name.startswith(("score_", "lse_", "select", "gather", "specpc_", "decode_", "colsum_")):
            continue
        f = sum(fetch[name]) / len(fetch[name])
        w = sum(write[name]) / len(write[name])
        kernels[name] = {"dispatches": len(fetch[name]), "fetch_kib_raw": round(f, 1), "write_kib_raw": round(w, 1),
                         "hbm_bytes_per_launch": round((f * f_scale + w * w_scale) * 1024.0)}
    return {"calibration": {"kernel": "torch.neg over fp32", "known_kib_each_way": known_kib,
                            "fetch_kib_raw": f_cal, "write_kib_raw": w_cal,
                            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
            "kernels": kernels}


SIMD_NUM = 1024  # 256 CUs x 4 SIMDs
XCD_NUM = 8      # rocprofv3's GRBM_GUI_ACTIVE here is the sum over the 8 XCDs' GRBM blocks


def dispatch_durations(d: str) -> dict[str, list[float]]:
    """Kernel duration (s) per dispatch of a counter-collection run, from its own timestamps."""
    dur, name_of = {}, {}
    with open(_csv(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            key = int(r["Dispatch_Id"])
            dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            name_of[key] = short_name(r["Kernel_Name"])
    out = collections.defaultdict(list)
    for key in sorted(dur):
        out[name_of[key]].append(dur[key])
    return out


def mfma_summary(d: str) -> list[dict]:
    """Per kernel: MFMA busy share of the SIMDs (SQ_VALU_MFMA_BUSY_CYCLES over the per-XCD
    GRBM_GUI_ACTIVE x SIMDs, as rocprofv3's MfmaUtil), executed bf16 MFMA flops
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), vector instructions, and the core clock (per-XCD
    GRBM_GUI_ACTIVE over the dispatch's duration)."""
    busy = per_dispatch(d, "SQ_VALU_MFMA_BUSY_CYCLES")
    mops = per_dispatch(d, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    valu = per_dispatch(d, "SQ_INSTS_VALU")
    gui = per_dispatch(d, "GRBM_GUI_ACTIVE")
    dur = dispatch_durations(d)
    mean = lambda v: sum(v) / len(v) if v else 0.0
    rows = []
    for name in sorted(busy):
        if not name.startswith(("score_", "specpc_", "decode_")) or name not in gui:
            continue
        g = mean(gui[name]) / XCD_NUM
        rows.append({"kernel": name, "dispatches": len(busy[name]),
                     "mfma_busy_pct": round(100.0 * mean(busy[name]) / (g * SIMD_NUM), 1),
                     "bf16_mfma_tflop": round(mean(mops.get(name, [])) * 512 / 1e12, 3),
                     "valu_insts": round(mean(valu.get(name, []))),
                     "ms": round(mean(dur[name]) * 1e3, 3),
                     "clock_ghz": round(g / mean(dur[name]) / 1e9, 2)})
    return rows


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--stats")
    p.add_argument("--fetch")
    p.add_argument("--write")
    p.add_argument("--calib-mib", type=int, default=0)
    p.add_argument("--workload", default="")
    p.add_argument("--title", default="")
    p.add_argument("--command", action="append", default=[])
    p.add_argument("--bench-log", help="log of the profiled bench.py run: its JSON line's event timings are listed")
    p.add_argument("--mfma", help="directory of a --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                                  "SQ_INSTS_VALU GRBM_GUI_ACTIVE run")
    p.add_argument("--out")
    a = p.parse_args(argv)
    if a.mfma:
        lines = [f"# {a.title}" if a.title else "# MFMA and vector counters per kernel", ""]
        lines += ["Command:", ""] + [f"    {c}" for c in a.command] + [""]
        lines.append(f"{'kernel':<40} {'calls':>5} {'ms':>8} {'MFMA busy %':>11} {'bf16 TFLOP':>10} {'VALU insts':>12} "
                     f"{'clock GHz':>9}")
        for r in mfma_summary(a.mfma):
            lines.append(f"{r['kernel'][:40]:<40} {r['dispatches']:>5} {r['ms']:>8} {r['mfma_busy_pct']:>11} "
                         f"{r['bf16_mfma_tflop']:>10} {r['valu_insts']:>12} {r['clock_ghz']:>9}")
        text = "\n".join(lines) + "\n"
    elif a.stats:
        lines = [f"# {a.title}" if a.title else "# rocprofv3 kernel statistics", ""]
        lines += ["Command:", ""] + [f"    {c}" for c in a.command] + [""]
        lines.append(f"{'kernel':<44} {'calls':>6} {'total ms':>10} {'avg us':>10} {'%':>6}")
        for r in stats_table(a.stats):
            lines.append(f"{r['name'][:44]:<44} {r['calls']:>6} {r['total_ms']:>10.3f} {r['avg_us']:>10.1f} "
                         f"{r['pct']:>6.2f}")
        if a.bench_log:
            bench = None
            with open(a.bench_log) as f:
                for line in f:
                    if line.startswith("{"):
                        bench = json.loads(line)
            if bench:
                lines += ["", "Same run, bench.py's own HIP-event timing per launch (launch stream):", ""]
                for k, v in bench.get("kernels", {}).items():
                    lines.append(f"    {k:<20} avg {v['avg_ms'] * 1e3:10.1f} us")
                lines.append(f"    step: {bench['ms_per_step']} ms; roofline {json.dumps(bench.get('roofline'))}")
        text = "\n".join(lines) + "\n"
    elif a.fetch and a.write:
        t = traffic(a.fetch, a.write, a.calib_mib)
        t.update({"workload": a.workload, "kernel_source_hash": kernel_source_hash(), "commands": a.command})
        text = json.dumps(t, indent=1) + "\n"
    else:
        p.error("give --stats DIR, --mfma DIR, or --fetch DIR --write DIR")
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
