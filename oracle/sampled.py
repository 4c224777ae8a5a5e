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
        # Every affinity core, up to the 16-core host share one GPU gets.
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


def _head_grad_rows(args):
    """Oracle backward work for sampled rows of one head: each row's routing
    and its softmax-attention gradient (dq for the row and its dk, dv
    contributions), with a seeded upstream gradient. Timing only."""
    w, b, h, ts = args
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    G = w.group
    k, v = synth.make_kv(w.seed, b, h // G, w.seq_len, w.head_dim, w.block_size, w.dtype)
    q = synth.make_q(w.seed, b, h, w.seq_len, w.head_dim, w.dtype)
    do = np.random.default_rng(np.random.SeedSequence([w.seed, 1000, b, h])).standard_normal(q.shape)
    t0 = time.perf_counter()
    kbar = moba.pool_keys(k, w.block_size, w.pooling)
    t1 = time.perf_counter()
    for t in ts:
        c = int(t) // w.block_size
        idx, _, _, _ = moba.select_blocks(q[t], kbar, c, w.top_k, w.causal)
        keys = moba.attended_keys(int(t), idx, w.block_size, w.causal, w.seq_len)
        moba.attend_grad(q[t], k, v, keys, do[t])
    return t1 - t0, time.perf_counter() - t1, len(ts)


def oracle_backward_rows(w: "synth.Workload", rows: np.ndarray, workers: int | None = None):
    """Times the oracle's backward on sampled rows (b, h, t); returns
    (pool_seconds, row_seconds, rows, heads, workers): one pooling pass per
    sampled head, and the rows' routing and gradients."""
    rows = np.asarray(rows, dtype=np.int64)
    groups = {}
    for b, h, t in rows:
        groups.setdefault((int(b), int(h)), []).append(int(t))
    jobs = [(w, b, h, np.array(ts, np.int64)) for (b, h), ts in groups.items()]
    if workers is None:
        # Every affinity core, up to the 16-core host share one GPU gets.
        workers = min(16, len(os.sched_getaffinity(0)))
    workers = max(1, min(workers, len(jobs)))
    if workers == 1:
        res = list(map(_head_grad_rows, jobs))
    else:
        import multiprocessing as mp
        with mp.get_context("fork").Pool(workers) as pool:
            res = pool.map(_head_grad_rows, jobs)
    return sum(r[0] for r in res), sum(r[1] for r in res), sum(r[2] for r in res), len(jobs), workers
