"""Oracle over seeded sampled rows of a named workload (test infrastructure).

Regenerates the inputs of each needed head from the workload's seed (it
never reads GPU buffers) and evaluates the fp64 oracle on the requested
query rows. Heads are spread over worker processes; each worker pins BLAS
to one thread.
"""
from __future__ import annotations

import os
import time

import numpy as np

import synth
from . import moba


def _head_rows(args):
    w, b, h, ts = args
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    t0 = time.perf_counter()
    G = w.group
    hk = h // G
    k, v = synth.make_kv(w.seed, b, hk, w.seq_len, w.head_dim, w.block_size, w.dtype)
    if w.gate_shared and G > 1:
        qs = np.stack([synth.make_q(w.seed, b, hk * G + g, w.seq_len, w.head_dim, w.dtype) for g in range(G)])
    else:
        qs = synth.make_q(w.seed, b, h, w.seq_len, w.head_dim, w.dtype)[None]
    t1 = time.perf_counter()
    moba.pool_keys(k, w.block_size, w.pooling)
    t2 = time.perf_counter()
    if len(qs) > 1:  # the group routes together; only head h's rows are kept
        res = moba.forward_group(qs, k, v, w.block_size, w.top_k, w.causal, rows=ts, pooling=w.pooling,
                                 shared_gate=True)[h % G]
    else:
        res = moba.forward_head(qs[0], k, v, w.block_size, w.top_k, w.causal, rows=ts, pooling=w.pooling)
    t3 = time.perf_counter()
    return b, h, ts, res, t1 - t0, t2 - t1, t3 - t2


def oracle_rows(w: "synth.Workload", rows: np.ndarray, workers: int | None = None):
    """rows: int64 [n, 3] of (b, h, t). Returns dict keyed like forward_head
    (o, idx, flag, a, b) in the order of `rows`, plus timing fields:
    gen_s (input regeneration), pool_s (one pooling pass per head) and
    oracle_s (pooling + the rows), summed over workers, plus heads, wall_s
    and workers."""
    rows = np.asarray(rows, dtype=np.int64)
    groups = {}
    for i, (b, h, t) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append((i, int(t)))
    jobs = [(w, b, h, np.array([t for _, t in lst], np.int64)) for (b, h), lst in groups.items()]
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    workers = max(1, min(workers, len(jobs)))
    n = len(rows)
    out = {"o": np.zeros((n, w.head_dim)), "idx": np.zeros((n, w.top_k), np.int64),
           "flag": np.zeros(n, bool), "a": np.zeros(n), "b": np.zeros(n)}
    gen_s = orc_s = pool_s = 0.0
    t0 = time.perf_counter()
    if workers == 1:
        results = map(_head_rows, jobs)
        pool = None
    else:
        import multiprocessing as mp
        pool = mp.get_context("fork").Pool(workers)
        results = pool.imap_unordered(_head_rows, jobs)
    try:
        for b, h, ts, res, g, p, o in results:
            gen_s += g
            pool_s += p
            orc_s += o
            for r, (i, _) in enumerate(groups[(b, h)]):
                for key in out:
                    out[key][i] = res[key][r]
    finally:
        if pool is not None:
            pool.close()
            pool.join()
    out["gen_s"] = gen_s
    out["oracle_s"] = orc_s
    out["pool_s"] = pool_s
    out["heads"] = len(jobs)
    out["wall_s"] = time.perf_counter() - t0
    out["workers"] = workers
    return out
