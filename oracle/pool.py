"""The fp64 oracle over many independent units in a process pool.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by the GPU parity
tests, to compare every (layer, head) unit of the full-size workloads, and by
bench.py's cpu_baseline leg, to time the oracle on the host's cores.

A unit is one (layer, KV head) of SpecKV (or one query head with one kept set
per query head), or one (layer, query head) map of SpecPC; units share
nothing, so they run side by side.  Workers are fresh interpreters (spawn:
nothing of the parent's state, and no device handle, is inherited), each with
one BLAS thread.  Inputs travel as raw element arrays (bfloat16 as its uint16
words, float32 as is) and are widened to float64 in the worker, exactly: both
formats are exact in float64.  The arithmetic is the oracle's own functions,
unchanged.
"""
from __future__ import annotations

import multiprocessing
import os
import time

import numpy as np

_BLAS_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def worker_count(cap: int = 16) -> int:
    """Workers for the pool: the cores this process may run on, at most `cap`."""
    return max(1, min(len(os.sched_getaffinity(0)), cap))


def exact_f64(raw) -> np.ndarray:
    """float64 copy of raw elements: uint16 arrays are bfloat16 bit patterns
    (widened by placing them in the top half of a float32), float32 as is."""
    raw = np.asarray(raw)
    if raw.dtype == np.uint16:
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if raw.dtype == np.float32:
        return raw.astype(np.float64)
    raise TypeError(f"raw elements must be uint16 (bfloat16 bits) or float32, not {raw.dtype}")


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _speckv_unit(t):
    """SpecKV scores of one unit (oracle.head_scores); with "step", also the
    pooling, selection and compaction of K and V, timed."""
    from .speckv import compact_rows, head_scores, pool1d, select_kept
    t0 = time.perf_counter()
    q, k = exact_f64(t["q"]), exact_f64(t["k"])
    s = head_scores(q, k[:t["n_pre"]], t["scale"], t.get("aggregation", "sum"))
    if not t.get("step"):
        return t["uid"], s, time.perf_counter() - t0
    kept = select_kept(pool1d(s, t["pool_kernel"], "max"), t["C_max"], t["n_window"])
    compact_rows(t["k"], kept)
    compact_rows(t["v"], kept)
    return t["uid"], None, time.perf_counter() - t0


def _specpc_maps(t):
    """Sum over a batch of (layer, query head) maps of the causal window
    probabilities on the input columns (oracle.causal_window_probabilities)."""
    from .specpc import causal_window_probabilities
    t0 = time.perf_counter()
    acc = None
    for q_raw, k_raw in t["maps"]:
        p = causal_window_probabilities(exact_f64(q_raw), exact_f64(k_raw), t["scale"])[:, :t["n_in"]]
        acc = p if acc is None else acc + p
    return t["uid"], acc, time.perf_counter() - t0


def _decode_units(t):
    """Decode attention of a batch of units (oracle.head_attention)."""
    from .decode import head_attention
    t0 = time.perf_counter()
    outs = [head_attention(exact_f64(q), exact_f64(k), exact_f64(v), t["scale"]) for q, k, v in t["units"]]
    return t["uid"], outs, time.perf_counter() - t0


_KINDS = {"speckv": _speckv_unit, "specpc_maps": _specpc_maps, "decode": _decode_units}


def _run(item):
    kind, task = item
    return _KINDS[kind](task)


class OraclePool:
    """A pool of spawned workers with one BLAS thread each.

        with OraclePool(n) as pool:
            for uid, result, seconds in pool.imap("speckv", tasks):
                ...

    `tasks` may be a generator (inputs are then produced while earlier units
    run); results arrive as units finish, each with its worker-side seconds.
    """

    def __init__(self, n_workers: int | None = None):
        self.n = n_workers or worker_count()
        saved = {k: os.environ.get(k) for k in _BLAS_ENV}
        for k in _BLAS_ENV:  # read by the workers' BLAS at import
            os.environ[k] = "1"
        try:
            self._pool = multiprocessing.get_context("spawn").Pool(self.n, initializer=_init_worker)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def imap(self, kind: str, tasks):
        return self._pool.imap_unordered(_run, ((kind, t) for t in tasks), chunksize=1)

    def close(self):
        self._pool.close()
        self._pool.join()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        if exc[0] is not None:
            self._pool.terminate()
            self._pool.join()
        else:
            self.close()
        return False
