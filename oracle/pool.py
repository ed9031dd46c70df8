"""Process-parallel runs of the CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the test-suite and the benchmark's
CPU-baseline leg may use this module; the GPU product path never does.

A task is (workload, seed, head, pathway, first query row, row count, box
radius, K/V scales).  The worker regenerates that head's seeded inputs with
the input generator (the module that also feeds the GPU tests, so both sides
see identical bits), for an fp8 cache (scales given) replaces K and V by the
oracle's E4M3 quantise-then-decode of them, and calls the oracle's plain
per-head attention, `attend_head`, on those rows.
Nothing here computes attention itself: the pool only spreads independent
(head, pathway, rows) pieces over processes, which the oracle's definition
allows because output rows are independent.

Workers are spawned (not forked: the parent may hold a GPU context) and each
runs its BLAS with one thread, so `procs` is also the number of cores used.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

_CACHE: dict = {}


def default_procs() -> int:
    """Worker processes: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _head_inputs(wl, seed, head, kv_scales=None):
    """(q, k, v) of one head as the oracle takes them, kept for the next task
    on the same head (tasks of one head arrive together).  With kv_scales =
    (k_scale, v_scale), K and V are the values an fp8 (E4M3) cache holds:
    the oracle's codes of x / scale, decoded and multiplied by the scale."""
    key = (wl, seed, head, kv_scales)
    if key not in _CACHE:
        from head_routed_kv_amd import workloads as W
        _CACHE.clear()
        data = W.window(wl, seed=seed, heads=[head], threads=1)
        q, k, v = (W.as_float(data[n], wl)[0] for n in ("q", "k", "v"))
        if kv_scales is not None:
            from oracle import headcast_oracle as O
            ks, vs = kv_scales
            k = O.dequantize_kv(O.quantize_kv(k, ks), ks)
            v = O.dequantize_kv(O.quantize_kv(v, vs), vs)
        _CACHE[key] = (q, k, v)
    return _CACHE[key]


def _run_task(task):
    from oracle import headcast_oracle as O
    wl, seed, head, pathway, r0, n, radius, kv_scales = task
    q, k, v = _head_inputs(wl, seed, head, kv_scales)
    g = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames, wl.cell_h, wl.cell_w)
    rows = np.arange(r0, r0 + n) if n > 0 else None
    t0 = time.perf_counter()
    out = O.attend_head(q, k, v, pathway, g, rows=rows, radius=radius)
    return task, out, time.perf_counter() - t0


def chunk_tasks(wl, seed, head_pathways, rows_per_task=None, radius=2, rows=None, kv_scales=None):
    """Tasks covering every query row (or the rows `rows`, one task per head)
    of each (head, pathway) pair, rows_per_task rows at a time."""
    tasks = []
    ks = None if kv_scales is None else (float(kv_scales[0]), float(kv_scales[1]))
    for h, pw in head_pathways:
        if rows is not None:
            tasks.append((wl, seed, int(h), int(pw), -1, 0, radius, ks))
            continue
        step = rows_per_task or wl.Nq
        for r0 in range(0, wl.Nq, step):
            tasks.append((wl, seed, int(h), int(pw), r0, min(step, wl.Nq - r0), radius, ks))
    return tasks


def _run_rows_task(task_rows):
    task, rows = task_rows
    from oracle import headcast_oracle as O
    wl, seed, head, pathway, _, _, radius, kv_scales = task
    q, k, v = _head_inputs(wl, seed, head, kv_scales)
    g = O.Geometry(wl.grid_h, wl.grid_w, wl.block_frames, wl.window_frames, wl.cell_h, wl.cell_w)
    t0 = time.perf_counter()
    out = O.attend_head(q, k, v, pathway, g, rows=np.asarray(rows), radius=radius)
    return task, out, time.perf_counter() - t0


def run(wl, seed, head_pathways, rows=None, rows_per_task=None, radius=2, procs=None, kv_scales=None):
    """Oracle outputs {(head, pathway): fp64 [rows, d]} for every pair in
    head_pathways, over all query rows (assembled from row chunks) or over
    the given rows; kv_scales = (k_scale, v_scale) attends over an fp8
    cache's decoded K/V.  Also returns the summed oracle seconds inside
    workers and the wall seconds of the pool run."""
    procs = procs or default_procs()
    tasks = chunk_tasks(wl, seed, head_pathways, rows_per_task, radius, rows, kv_scales)
    pieces: dict = {}
    cpu_s = 0.0
    t0 = time.perf_counter()
    # a worker that dies raises BrokenProcessPool here instead of hanging
    with ProcessPoolExecutor(min(procs, len(tasks)), mp_context=mp.get_context("spawn"),
                             initializer=_init_worker) as ex:
        if rows is not None:
            it = ex.map(_run_rows_task, [(t, list(map(int, rows))) for t in tasks])
        else:   # tasks of one head are consecutive; pairs of them share one input draw
            it = ex.map(_run_task, tasks, chunksize=2)
        last = t0
        for i, (task, out, sec) in enumerate(it):
            pieces.setdefault((task[2], task[3]), []).append((task[4], out))
            cpu_s += sec
            if time.perf_counter() - last > 20:   # a line per finished batch, at most every 20 s
                last = time.perf_counter()
                print(f"oracle pool: {i + 1}/{len(tasks)} pieces done", file=sys.stderr, flush=True)
    wall = time.perf_counter() - t0
    result = {}
    for key, parts in pieces.items():
        parts.sort(key=lambda x: x[0])
        result[key] = np.concatenate([p for _, p in parts], axis=0)
    return result, cpu_s, wall
