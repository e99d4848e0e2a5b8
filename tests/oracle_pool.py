"""Run the oracle comparisons of many (sequence, head) pairs in a pool of
host processes.

The oracle stays the plain per-pair code of ``oracle/``; the pool only runs
independent pairs side by side, so the full-size parity tests can compare
every pair of a 32k workload (the INT8 oracle takes about 1.4 s per 32768-token
pair on one core).  Workers are started with "spawn": they are fresh Python
processes that import NumPy and the oracle, never torch or the HIP library,
and never touch the GPU.  Each task carries the input bits of one pair and
the GPU's results for it, and runs the comparison functions of
``tests/parity_checks.py``; a failed comparison raises in the worker and is
re-raised in the test with its message.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

if mp.parent_process() is not None:  # a pool worker: one BLAS thread each
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"

import numpy as np  # noqa: E402

from oracle import attention, bits  # noqa: E402
from tests import parity_checks as pc  # noqa: E402

MAX_WORKERS = 16  # the host CPU share of one GPU on the test machines


def workers() -> int:
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))


def rows_task(a):
    """bf16 / fp32 rows: out of one pair vs masked full-history attention."""
    kb, vb, qb, n, W, out, what = a
    k64, v64, q64 = bits.to_f64(kb), bits.to_f64(vb), bits.to_f64(qb)
    ref = attention.masked_attention(q64, np.arange(n), k64[:n], v64[:n], n - 1, W)
    return pc.assert_close(out, ref, what)


def int8_task(a):
    """INT8: output and bounds of one pair (and its store when given)."""
    kb, vb, qb, n, W, b, h, out, cmax, c_all, store, what = a
    k64, v64, q64 = bits.to_f64(kb), bits.to_f64(vb), bits.to_f64(qb)
    if store is not None:
        pc.check_int8_store_arrays(*store, k64, v64, n, W, f"{what} b={b} h={h}")
    return pc.check_int8_decode(out, cmax, c_all, b, h, q64, k64, v64, n, W, what)


def dither_task(a):
    """Tier B: output, certificate, tv and gate of one pair."""
    kb, vb, qb, n, W, b, h, out, cert, tv, gate, req, layer, delta, what = a
    k64, v64, q64 = bits.to_f64(kb), bits.to_f64(vb), bits.to_f64(qb)
    return pc.check_dither_decode(out, cert, b, h, q64, k64, v64, n, W, req, layer, delta, tv, gate, what=what)


def run(fn, tasks, label: str, timeout: float = 600.0) -> float:
    """Run ``fn`` over ``tasks`` in the pool; prints progress about every 20
    seconds and returns the largest value the tasks return (the worst
    output error).  Raises if the pairs are not all checked within
    ``timeout`` seconds."""
    tasks = list(tasks)
    worst, done, t0, last = 0.0, 0, time.time(), time.time()
    print(f"{label}: {len(tasks)} pairs on {workers()} host processes", flush=True)
    pool = ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"))
    try:
        for r in pool.map(fn, tasks, chunksize=1, timeout=timeout):
            worst = max(worst, float(r))
            done += 1
            if time.time() - last > 20 or done == len(tasks):
                print(f"{label}: {done}/{len(tasks)} pairs checked, {time.time() - t0:.0f} s, "
                      f"worst abs err {worst:.2e}", flush=True)
                sys.stdout.flush()
                last = time.time()
    finally:
        pool.shutdown(wait=False, cancel_futures=True)
    return worst
