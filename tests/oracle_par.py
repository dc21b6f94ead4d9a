"""Runs the CPU oracle's row-range and column-set functions on the host's cores.

Test infrastructure: it only splits the work (disjoint row ranges, disjoint
column sets) over a thread pool with one BLAS thread per task, and stitches
the results together; every number comes from oracle.ref unchanged.  numpy
releases the interpreter lock inside its matrix products and element-wise
kernels, so the threads run in parallel."""
from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import ref


def _f64(x):
    x = np.asarray(x)
    return ref.bf16_to_f64(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float64)


def host_threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _pool_map(fn, tasks, progress=None):
    from threadpoolctl import threadpool_limits
    out = [None] * len(tasks)
    t0 = time.time()
    with threadpool_limits(1), ThreadPoolExecutor(host_threads()) as ex:
        futs = {ex.submit(fn, t): i for i, t in enumerate(tasks)}
        done = 0
        for f in futs:
            out[futs[f]] = f.result()
            done += 1
            if progress and (done % max(1, len(tasks) // 8) == 0 or done == len(tasks)):
                progress(f"oracle {done}/{len(tasks)} tasks, {time.time() - t0:.0f}s")
    return out


def row_stats(q, k, v, do, pos, r0, r1, softmax_scale=None, rows_per_task=512, progress=None):
    """ref.attn_row_stats over [r0, r1), in row ranges on the thread pool.
    Returns lse [hq][R], o [R][hq][d], D [hq][R]."""
    q, k, v, do = (_f64(a) for a in (q, k, v, do))
    # long rows cost more: cut the range into many tasks so the pool stays busy
    bounds = list(range(r0, r1, rows_per_task)) + [r1]
    tasks = list(zip(bounds[:-1], bounds[1:]))[::-1]        # longest rows first
    res = _pool_map(lambda t: ref.attn_row_stats(q, k, v, do, pos, t[0], t[1],
                                                 softmax_scale=softmax_scale), tasks, progress)
    res = res[::-1]
    lse = np.concatenate([r[0] for r in res], axis=1)
    o = np.concatenate([r[1] for r in res], axis=0)
    D = np.concatenate([r[2] for r in res], axis=1)
    return lse, o, D


def rows(q, k, v, do, pos, sel_rows, softmax_scale=None, per_task=32, progress=None):
    """ref.attn_rows for the given rows, split into row sets on the thread pool."""
    q, k, v, do = (_f64(a) for a in (q, k, v, do))
    sel_rows = np.asarray(sel_rows, np.int64)
    tasks = [sel_rows[i:i + per_task] for i in range(0, sel_rows.size, per_task)]
    res = _pool_map(lambda rr: ref.attn_rows(q, k, v, do, pos, rr, softmax_scale=softmax_scale),
                    tasks, progress)
    return (np.concatenate([r[0] for r in res], axis=0), np.concatenate([r[1] for r in res], axis=1),
            np.concatenate([r[2] for r in res], axis=0))


def key_cols(q, k, v, do, pos, cols, lse, D, softmax_scale=None, per_task=32, progress=None):
    """ref.attn_key_cols_from_stats for the given (sorted) key columns, split into
    consecutive column sets on the thread pool."""
    q, k, v, do = (_f64(a) for a in (q, k, v, do))
    cols = np.asarray(cols, np.int64)
    tasks = [cols[i:i + per_task] for i in range(0, cols.size, per_task)]
    res = _pool_map(lambda cc: ref.attn_key_cols_from_stats(q, k, v, do, pos, cc, lse, D,
                                                            softmax_scale=softmax_scale),
                    tasks, progress)
    return np.concatenate([r[0] for r in res], axis=0), np.concatenate([r[1] for r in res], axis=0)
