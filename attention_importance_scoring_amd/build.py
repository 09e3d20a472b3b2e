"""Builds libspeckv.so (the HIP kernels and the C ABI) in-tree for gfx950.

Each csrc/*.hip source is compiled by hipcc to an object file (in parallel),
then linked into attention_importance_scoring_amd/libspeckv.so.  Always
rebuilds: the call is also the "does it build" check.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libspeckv.so")
PEAKS_SRC = os.path.join(PKG_DIR, "peaks", "peaks.hip")
PEAKS_BIN = os.path.join(PKG_DIR, "peaks", "skv_peaks")  # measured unit ceilings, a separate program
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in (r.stderr or "").splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    workers = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(sources)} sources")
    build_peaks(verbose)
    return LIB_PATH


def build_peaks(verbose: bool = True) -> str:
    tmp = PEAKS_BIN + ".tmp"
    r = subprocess.run([hipcc(), *[f for f in HIPCC_FLAGS if f != "-fPIC"], PEAKS_SRC, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PEAKS_SRC}:\n{r.stderr}")
    os.replace(tmp, PEAKS_BIN)
    if verbose:
        print(f"built {PEAKS_BIN}")
    return PEAKS_BIN


if __name__ == "__main__":
    build()
