"""Seeded synthetic inputs for the MoBA prefill forward.

This module is shared by the CPU oracle and by the GPU path (tests, bench).
It holds no part of MoBA's arithmetic: it only draws Q, K and V and picks
which query rows a sampled check visits.

Recipe (one per named workload):
  * q and v are standard normal;
  * k is standard normal plus one bias vector per (batch, head, key block),
    drawn from N(0, 0.5^2) and shared by every token of that block, which
    spreads the block means apart so that block selection is not decided
    by noise alone;
  * values are produced in float32; for bf16 workloads they are then
    rounded to bf16 (round to nearest, ties to even) and both sides read
    those exact values.

Streams: tensor id (q=0, k noise=1, k bias=2, v=3) and (b, h) seed a
numpy PCG64 generator through SeedSequence([seed, id, b, h]), so any head
can be regenerated on its own.
"""
from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np

TENSOR_Q, TENSOR_KNOISE, TENSOR_KBIAS, TENSOR_V = 0, 1, 2, 3
ROW_SAMPLE_STREAM = 99


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    block_size: int
    top_k: int
    causal: bool
    dtype: str  # "f32" or "bf16"
    seed: int
    pooling: str = "mean"  # block summary the gate scores: "mean", "max" or "mean+max"
    kv_heads: int = 0      # key/value heads (grouped-query attention); 0 = heads
    gate_shared: bool = False  # a group of query heads routes on its summed scores

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block_size)

    @property
    def kvh(self) -> int:
        return self.kv_heads or self.heads

    @property
    def group(self) -> int:
        return self.heads // self.kvh


# The five named workloads (sizes of the pages' settings: block 512 / top-k 3
# at 32K, block 2048 / top-k 3 at 32K, block 4096 / top-k 4 at 128K, and 1M).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 2048, 64, 256, 3, True, "f32", 0),
    "headline_32k": Workload("headline_32k", 1, 32, 32768, 128, 512, 3, True, "bf16", 1),
    "coarse_32k": Workload("coarse_32k", 1, 32, 32768, 128, 2048, 3, True, "bf16", 2),
    "long_128k": Workload("long_128k", 1, 32, 131072, 128, 4096, 4, True, "bf16", 3),
    "long_1m": Workload("long_1m", 1, 32, 1048576, 128, 512, 3, True, "bf16", 4),
}
WORKLOAD_ORDER = ["tiny", "headline_32k", "coarse_32k", "long_128k", "long_1m"]
# The headline inputs (same seed, same tensors) gated by the other block
# summaries the serving article names next to the mean.
WORKLOADS["headline_32k_max"] = Workload("headline_32k_max", 1, 32, 32768, 128, 512, 3, True, "bf16", 1, "max")
WORKLOADS["headline_32k_meanmax"] = Workload("headline_32k_meanmax", 1, 32, 32768, 128, 512, 3, True, "bf16", 1,
                                             "mean+max")
POOLING_VARIANTS = ["headline_32k_max", "headline_32k_meanmax"]
# 32768 + 256 tokens: 65 blocks of 512, the last one holding 256.
WORKLOADS["headline_33k_short_block"] = Workload("headline_33k_short_block", 1, 32, 33024, 128, 512, 3, True,
                                                 "bf16", 5)
SHAPE_VARIANTS = ["headline_33k_short_block"]
# Grouped-query attention at the headline shape: 32 query heads over 8
# key/value heads, each query head routing on its own or each group of four
# routing once on its summed scores.
WORKLOADS["headline_32k_gqa4"] = Workload("headline_32k_gqa4", 1, 32, 32768, 128, 512, 3, True, "bf16", 6,
                                          kv_heads=8)
WORKLOADS["headline_32k_gqa4_shared"] = Workload("headline_32k_gqa4_shared", 1, 32, 32768, 128, 512, 3, True,
                                                 "bf16", 6, kv_heads=8, gate_shared=True)
GQA_VARIANTS = ["headline_32k_gqa4", "headline_32k_gqa4_shared"]


def _rng(seed: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, b, h])))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16-representable float32 values -> their 16-bit patterns (int16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x


def make_q(seed: int, b: int, h: int, seq_len: int, head_dim: int, dtype: str):
    """q of query head (b, h), float32 [seq_len, head_dim]."""
    q = _rng(seed, TENSOR_Q, b, h).standard_normal((seq_len, head_dim), dtype=np.float32)
    return _cast(q, dtype)


def make_kv(seed: int, b: int, h: int, seq_len: int, head_dim: int, block_size: int, dtype: str):
    """(k, v) of key/value head (b, h), each float32 [seq_len, head_dim]."""
    S, D = seq_len, head_dim
    nb = -(-S // block_size)  # a short last block gets its own bias too
    kn = _rng(seed, TENSOR_KNOISE, b, h).standard_normal((S, D), dtype=np.float32)
    bias = _rng(seed, TENSOR_KBIAS, b, h).normal(0.0, 0.5, (nb, D)).astype(np.float32)
    kn += np.repeat(bias, block_size, axis=0)[:S]
    v = _rng(seed, TENSOR_V, b, h).standard_normal((S, D), dtype=np.float32)
    return _cast(kn, dtype), _cast(v, dtype)


def make_head(seed: int, b: int, h: int, seq_len: int, head_dim: int,
              block_size: int, dtype: str):
    """Return (q, k, v), each float32 [seq_len, head_dim], for one (b, h)."""
    q = make_q(seed, b, h, seq_len, head_dim, dtype)
    return (q, *make_kv(seed, b, h, seq_len, head_dim, block_size, dtype))


def make_group(w: "Workload", b: int, hk: int):
    """(q [group, S, D] of the query heads hk * group .. + group - 1, k, v of
    key/value head hk). With kv_heads = heads this is make_head of (b, hk)."""
    G = w.group
    q = np.stack([make_q(w.seed, b, hk * G + g, w.seq_len, w.head_dim, w.dtype) for g in range(G)])
    k, v = make_kv(w.seed, b, hk, w.seq_len, w.head_dim, w.block_size, w.dtype)
    return q, k, v


def make_inputs(w: Workload, heads=None):
    """Full [B, H, S, D] float32 tensors (bf16-valued for bf16 workloads).

    heads: optional list of (b, h) to fill; other heads are left zero.
    Intended for workloads that fit comfortably in host memory.
    """
    shape = (w.batch, w.heads, w.seq_len, w.head_dim)
    q = np.zeros(shape, np.float32)
    k = np.zeros(shape, np.float32)
    v = np.zeros(shape, np.float32)
    todo = heads if heads is not None else [(b, h) for b in range(w.batch) for h in range(w.heads)]
    for b, h in todo:
        q[b, h], k[b, h], v[b, h] = make_head(w.seed, b, h, w.seq_len, w.head_dim, w.block_size, w.dtype)
    return q, k, v


def _head_job(args):
    w, b, h = args
    q, k, v = make_head(w.seed, b, h, w.seq_len, w.head_dim, w.block_size, w.dtype)
    if w.dtype == "bf16":
        return b, h, bf16_bits(q), bf16_bits(k), bf16_bits(v)
    return b, h, q, k, v


def _group_job(args):
    w, b, hk = args
    q, k, v = make_group(w, b, hk)
    if w.dtype == "bf16":
        return b, hk, bf16_bits(q), bf16_bits(k), bf16_bits(v)
    return b, hk, q, k, v


def iter_groups_parallel(w: Workload, workers: int | None = None):
    """Yield (b, hk, q [group, S, D], k, v) per key/value head, generated in
    worker processes (bf16 workloads as int16 bit patterns, like
    iter_heads_parallel)."""
    jobs = [(w, b, hk) for b in range(w.batch) for hk in range(w.kvh)]
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if workers <= 1 or len(jobs) == 1:
        for j in jobs:
            yield _group_job(j)
        return
    import multiprocessing as mp
    with mp.get_context("fork").Pool(workers) as pool:
        for out in pool.imap(_group_job, jobs, chunksize=1):
            yield out


def iter_heads_parallel(w: Workload, workers: int | None = None):
    """Yield (b, h, q, k, v) per head, generated in worker processes.

    For bf16 workloads the arrays are int16 bit patterns (ready to view as
    bf16); for f32 workloads they are float32. Heads arrive in (b, h) order.
    """
    jobs = [(w, b, h) for b in range(w.batch) for h in range(w.heads)]
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if workers <= 1 or len(jobs) == 1:
        for j in jobs:
            yield _head_job(j)
        return
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        for out in pool.imap(_head_job, jobs, chunksize=1):
            yield out


def sample_rows(w: Workload, n: int = 4096) -> np.ndarray:
    """Seeded sample of query rows, int64 [n, 3] of (b, h, t), sorted.

    Always contains the edge rows: t = 0, Bs-1, Bs, S-1 and the first and
    last token of the last block, on the first and the last head.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, ROW_SAMPLE_STREAM])))
    Bs, S = w.block_size, w.seq_len
    edges_t = sorted({0, Bs - 1, min(Bs, S - 1), (w.n_blocks - 1) * Bs, S - 1})
    forced = []
    for b in {0, w.batch - 1}:
        for h in {0, w.heads - 1}:
            forced += [(b, h, t) for t in edges_t]
    forced = sorted(set(forced))
    total = w.batch * w.heads * S
    if n >= total:
        flat = np.arange(total, dtype=np.int64)
    else:
        chosen = set(((b * w.heads + h) * S + t) for b, h, t in forced)
        need = n - len(chosen)
        draw = rng.choice(total, size=min(total, need * 2 + 64), replace=False)
        for x in draw:
            if need == 0:
                break
            if int(x) not in chosen:
                chosen.add(int(x))
                need -= 1
        flat = np.array(sorted(chosen), dtype=np.int64)
    b = flat // (w.heads * S)
    h = (flat // S) % w.heads
    t = flat % S
    return np.stack([b, h, t], axis=1)
