"""The fp64 oracle over row ranges in spawned worker processes, for the
full-size parity checks (test infrastructure).

Key-side gradients at full size need the whole score row of every query that
sees the sampled keys (up to 32768 rows x 32768 keys per head); numpy's
element-wise passes run on one core, so the rows are split into ranges and
each range is handed to a worker.  Each worker draws the workload's seeded
inputs itself (the generators are deterministic) and calls the oracle's own
``dkv_keys`` / ``dq_rows`` on its range; dK and dV over all rows are the sums
of the per-range results, which is their definition (a sum over rows).
Workers are spawned, not forked, so they share no GPU state with the test
process, and they never touch the GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

_HOST = {}


def worker_count() -> int:
    """Worker processes: the process's CPU share (capped by OMP_NUM_THREADS
    where that is set), at most 8."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(8, n))


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass


def _host(w):
    key = (w.name, w.seed, w.B, w.Hq, w.Hkv, w.L, w.D)
    if key not in _HOST:
        from workloads import make_inputs, to_f64, to_i32
        inp = make_inputs(w)
        _HOST.clear()
        _HOST[key] = dict(q=to_f64(inp["q"]), k=to_f64(inp["k"]), v=to_f64(inp["v"]),
                          do=to_f64(inp["do"]), temp=to_f64(inp["temperature"]),
                          seg=to_i32(inp["segment_ids"]), rb=to_i32(inp["ranker_bounds"]))
    return _HOST[key]


def _params(w):
    from oracle import Params
    return Params(w.sm_scale, w.causal, w.window_len, w.cap_method, w.cap, w.alpha, w.beta,
                  w.z_loss_weight)


def _dkv_part(w, b, g, keys, rows):
    from oracle import dkv_keys
    h = _host(w)
    r = dkv_keys(h["q"], h["k"], h["v"], h["do"], _params(w), b, g, keys, h["temp"], h["seg"],
                 h["rb"], rows=rows)
    return r["dk"], r["dv"]


def _dq_part(w, b, hq, rows):
    from oracle import dq_rows
    h = _host(w)
    return dq_rows(h["q"], h["k"], h["v"], h["do"], _params(w), b, hq, rows, h["temp"], h["seg"],
                   h["rb"])


def _pool(n):
    return cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                                  initializer=_init)


def dkv_keys_pooled(w, jobs, say=print, part_rows: int = 2048):
    """jobs: list of (b, g, keys, rows).  Returns one dict(dk, dv) per job, each
    the oracle's dK / dV of those keys summed over the given rows (all rows
    that can see the keys)."""
    tasks = []
    for j, (b, g, keys, rows) in enumerate(jobs):
        rows = np.asarray(rows)
        for a in range(0, len(rows), part_rows):
            tasks.append((j, b, g, np.asarray(keys), rows[a:a + part_rows]))
    out = [None] * len(jobs)
    n = worker_count()
    say(f"  oracle: {len(tasks)} row ranges over {n} workers")
    with _pool(n) as ex:
        futs = {ex.submit(_dkv_part, w, b, g, keys, rows): j for j, b, g, keys, rows in tasks}
        done = 0
        for f in cf.as_completed(futs):
            j = futs[f]
            dk, dv = f.result()
            if out[j] is None:
                out[j] = dict(dk=dk.copy(), dv=dv.copy())
            else:
                out[j]["dk"] += dk
                out[j]["dv"] += dv
            done += 1
            if done % max(1, len(tasks) // 8) == 0 or done == len(tasks):
                say(f"  oracle: {done}/{len(tasks)} row ranges")
    return out


def dq_rows_pooled(w, jobs, say=print):
    """jobs: list of (b, hq, rows).  Returns the oracle's dq_rows dict per job."""
    with _pool(worker_count()) as ex:
        res = list(ex.map(_dq_part, [w] * len(jobs), [j[0] for j in jobs], [j[1] for j in jobs],
                          [np.asarray(j[2]) for j in jobs]))
    say(f"  oracle: {len(jobs)} row sets")
    return res
