"""Run the oracle over (request, head) units on a process pool, for timing only.

TEST INFRASTRUCTURE ONLY (see the package docstring). The arithmetic is the
oracle's own (``attention.varlen_paged`` / ``attention.prefill_varlen``); this
module only splits the unit list across forked worker processes, each with a
single BLAS thread, and reassembles the rows.
"""

import multiprocessing as mp
import os
import time

import numpy as np

from . import attention

_JOB = {}


def _worker(chunk):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)        # one BLAS thread per worker process
    except Exception:                      # threadpoolctl missing: run with whatever BLAS uses
        pass
    kind, args, kwargs = _JOB["kind"], _JOB["args"], _JOB["kwargs"]
    fn = attention.varlen_paged if kind == "paged" else attention.prefill_varlen
    out, lse = fn(*args, units=chunk, **kwargs)
    rows = []
    cu = _JOB["cu"]
    for b, h in chunk:
        lo, hi = cu[b], cu[b + 1]
        rows.append((b, h, out[lo:hi, h].copy(), lse[lo:hi, h].copy()))
    return rows


def run_units(kind, args, kwargs, units, cu, out_shape, lse_shape, workers=None):
    """kind: "paged" (varlen_paged positional args) or "prefill" (prefill_varlen args).

    Returns (out, lse, wall_seconds, workers_used); rows outside ``units`` are NaN.
    """
    workers = max(1, int(workers or os.cpu_count() or 1))
    units = [(int(b), int(h)) for b, h in units]
    _JOB.update(kind=kind, args=args, kwargs=kwargs, cu=[int(x) for x in cu])
    # contiguous slices, so that the query heads of one KV head stay in one worker and share
    # its gathered pages
    per = -(-len(units) // workers)
    chunks = [units[i:i + per] for i in range(0, len(units), per)]
    chunks = [c for c in chunks if c]
    out = np.full(out_shape, np.nan)
    lse = np.full(lse_shape, np.nan)
    t0 = time.perf_counter()
    if len(chunks) == 1:
        results = [_worker(chunks[0])]
    else:
        with mp.get_context("fork").Pool(len(chunks)) as pool:
            results = pool.map(_worker, chunks)
    wall = time.perf_counter() - t0
    for rows in results:
        for b, h, o, l in rows:
            lo, hi = _JOB["cu"][b], _JOB["cu"][b + 1]
            out[lo:hi, h] = o
            lse[lo:hi, h] = l
    return out, lse, wall, len(chunks)
