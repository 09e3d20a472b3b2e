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


def per_dispatch(d: str, counter: str) -> dict[str, list[float]]:
    """Counter value (summed over the dimensions rocprofv3 reports) per dispatch, grouped by kernel."""
    by_dispatch = collections.defaultdict(float)
    name_of = {}
    with open(_csv(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            by_dispatch[key] += float(r["Counter_Value"])
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
    p.add_argument("--out")
    a = p.parse_args(argv)
    if a.stats:
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
        p.error("give --stats DIR, or --fetch DIR --write DIR")
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
