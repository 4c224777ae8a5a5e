#!/usr/bin/env python3
"""MoBA prefill forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole MoBA forward (pool -> gate/top-k -> varlen pack ->
past-block attention -> own-block attention and merge) over one batch of
seeded synthetic Q/K/V already resident in HBM. Prints one JSON line:
throughput in tokens/s, effective TFLOP/s of the algorithmic work, the
roofline of the dominant kernel (HIP-event durations of its launches inside
the timed region), the speedup over the library's dense causal kernel, and
the CPU fp64 oracle timed on a bounded sample of the same workload. The
line's `long_context` list repeats the GPU measurements (not the CPU
baseline) at 128K and 1M tokens, the other lengths the metric is quoted
at, on inputs drawn on the device with the same distribution; its
`backward` entry times moba_backward on the main workload's inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (MFMA and vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoBA fwd tokens/sec + effective TFLOP/s (% bf16 MFMA peak) at 32K/128K/1M"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def work_model(w):
    """Algorithmic work of one forward, counted from MoBA's definition:
    gate 2*D flops per (query, eligible past block); attention 4*D flops per
    (query, attended key), split into past blocks and the own block. A gate
    shared by a group of query heads scores the group's summed query once
    per (query position, block); pooling reads K once per key/value head."""
    S, D, Bs, nb, bh = w.seq_len, w.head_dim, w.block_size, w.n_blocks, w.batch * w.heads
    bhkv = w.batch * w.kvh
    gate_rows = bhkv if w.gate_shared else bh
    k_eff = min(w.top_k, nb)
    gate_pairs = past_pairs = own_keys = 0
    for c in range(nb):
        n = min(Bs, S - c * Bs)  # queries in block c (a short last block holds fewer)
        elig = c if w.causal else nb - 1
        gate_pairs += n * elig
        past_pairs += n * min(k_eff - 1, elig)  # causal past blocks are whole blocks of Bs keys
        own_keys += n * (n + 1) // 2 if w.causal else n * n
    dense_keys = S * (S + 1) // 2 if w.causal else S * S
    esz = 2 if w.dtype == "bf16" else 4
    return {
        "gate_flops": gate_rows * 2 * D * gate_pairs,
        "past_flops": bh * 4 * D * past_pairs * Bs,
        "own_flops": bh * 4 * D * own_keys,
        "dense_flops": bh * 4 * D * dense_keys,
        "past_pairs": bh * past_pairs,
        "attended_keys": bh * (past_pairs * Bs + own_keys),
        "dense_keys": bh * dense_keys,
        "k_bytes": bhkv * S * D * esz,
        "qkvo_bytes": 2 * (bh + bhkv) * S * D * esz,
    }


def kernel_units(w, wm):
    """(bound, algorithmic work per launch, unit) for each library kernel."""
    D, bhkv, nb = w.head_dim, w.batch * w.kvh, w.n_blocks
    return {
        "gather_attn": ("mfma", wm["past_flops"], "flop"),
        "diag_merge": ("mfma", wm["own_flops"], "flop"),
        "gate_topk": ("mfma", wm["gate_flops"], "flop"),
        # K read once; the pooled keys written as fp64, fp32 and a bf16 pair.
        "pool": ("hbm", wm["k_bytes"] + bhkv * nb * D * (8 + 4 + 2 + 2), "byte"),
        "dense_attn": ("mfma", wm["dense_flops"], "flop"),
    }


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gather_attn": ["sparse_long_context_moba_amd/csrc/attn.hip", "sparse_long_context_moba_amd/csrc/engine.h",
                    "sparse_long_context_moba_amd/csrc/common.h"],
    "diag_merge": ["sparse_long_context_moba_amd/csrc/attn.hip", "sparse_long_context_moba_amd/csrc/engine.h",
                   "sparse_long_context_moba_amd/csrc/common.h"],
    "gate_topk": ["sparse_long_context_moba_amd/csrc/gate.hip", "sparse_long_context_moba_amd/csrc/common.h"],
    "pool": ["sparse_long_context_moba_amd/csrc/pool.hip", "sparse_long_context_moba_amd/csrc/common.h"],
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    text = open(path).read()
    m = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    d = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    if not m or not d or d.group(1) != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return float(m.group(1))


def upload(w, torch, workers=None):
    """q [B, H, S, D] and k, v [B, kv_heads, S, D], generated per key/value
    head and its group of query heads."""
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    G = w.group
    q = torch.empty((w.batch, w.heads, w.seq_len, w.head_dim), dtype=tdt, device="cuda")
    k, v = (torch.empty((w.batch, w.kvh, w.seq_len, w.head_dim), dtype=tdt, device="cuda") for _ in range(2))
    cast = (lambda t: t.view(torch.bfloat16)) if w.dtype == "bf16" else (lambda t: t)
    for b, hk, qh, kh, vh in synth.iter_groups_parallel(w, workers):
        q[b, hk * G:(hk + 1) * G].copy_(cast(torch.from_numpy(qh)))
        k[b, hk].copy_(cast(torch.from_numpy(kh)))
        v[b, hk].copy_(cast(torch.from_numpy(vh)))
    torch.cuda.synchronize()
    return q, k, v


def upload_device(w, torch, seed):
    """q, v ~ N(0,1) and k = N(0,1) + a per-(b, kv head, block) N(0, 0.5^2)
    bias shared by the block's tokens: the recipe's distribution, drawn on
    the device by torch's seeded generator (used where generating the
    seeded host streams would take minutes: the long-context sub-results)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    B, S, D, Bs, nb = w.batch, w.seq_len, w.head_dim, w.block_size, w.n_blocks
    q = torch.randn(B, w.heads, S, D, device="cuda", generator=g).to(dt)
    k = torch.empty(B, w.kvh, S, D, dtype=dt, device="cuda")
    for hk in range(w.kvh):  # one key/value head at a time bounds the fp32 temporaries
        kk = torch.randn(B, nb * Bs, D, device="cuda", generator=g).view(B, nb, Bs, D)
        kk += 0.5 * torch.randn(B, nb, 1, D, device="cuda", generator=g)
        k[:, hk] = kk.view(B, nb * Bs, D)[:, :S].to(dt)
        del kk
    v = torch.randn(B, w.kvh, S, D, device="cuda", generator=g).to(dt)
    torch.cuda.synchronize()
    return q, k, v


def time_forward(w, q, k, v, moba, torch, steps, warmup):
    """ms per forward and per-kernel average ms (HIP events on the stream)."""
    p = moba.problem(q, w.block_size, w.top_k, w.causal, w.pooling, w.kvh, w.gate_shared)
    ws = torch.empty(moba.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    idx = torch.empty((w.batch, w.heads, w.seq_len, w.top_k), dtype=torch.int32, device="cuda")

    def step():
        moba.forward(q, k, v, w.block_size, w.top_k, w.causal, out=o, idx=idx, workspace=ws, pooling=w.pooling,
                     gate_shared=w.gate_shared)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    with moba.timing() as tm:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    del ws, o, idx
    return 1e3 * elapsed / steps, {n: {"launches": c, "avg_ms": tot / c, "total_ms": tot} for n, c, tot in tm.rows}


def roofline_of(w, wm, kern, peak):
    """Roofline entry of the kernel with the largest time (algorithmic work
    per launch over its average launch duration)."""
    units = kernel_units(w, wm)
    dom = max((n for n in kern if n in units), key=lambda n: kern[n]["total_ms"])
    bound, work, unit = units[dom]
    avg_s = kern[dom]["avg_ms"] * 1e-3
    if bound == "hbm":
        achieved, rpeak, runit = work / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, rpeak, runit = work / avg_s / 1e12, peak, "TFLOP/s"
    return {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": rpeak, "unit": runit,
            "frac": round(achieved / rpeak, 4), "traffic": measured_traffic(dom, w.name),
            "work_per_launch": work, "work_unit": unit, "avg_launch_ms": round(kern[dom]["avg_ms"], 4)}


def long_context_result(name, args, moba, torch):
    """One sub-result of the long-context workloads the metric is quoted at
    (128K and 1M tokens): the same measurements as the main line, on
    device-drawn inputs of the recipe's distribution."""
    w = synth.WORKLOADS[name]
    wm = work_model(w)
    t0 = time.time()
    q, k, v = upload_device(w, torch, 1000 + w.seed)
    log(f"{name}: inputs drawn on the device in {time.time() - t0:.1f}s")
    ms, kern = time_forward(w, q, k, v, moba, torch, args.long_steps, 1)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    flops = wm["gate_flops"] + wm["past_flops"] + wm["own_flops"]
    ag_ms = sum(kern[n]["avg_ms"] for n in ("gate_topk", "gather_attn", "diag_merge") if n in kern)
    res = {
        "workload": name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len, "block_size": w.block_size,
        "top_k": w.top_k, "steps": args.long_steps, "ms_per_step": round(ms, 3),
        "tokens_per_s": round(w.batch * w.seq_len / (ms * 1e-3), 1),
        "effective_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "pct_peak": round(100 * flops / (ms * 1e-3) / 1e12 / peak, 2),
        "attn_gate_kernels_pct_peak": round(100 * flops / (ag_ms * 1e-3) / 1e12 / peak, 2),
        "kernels_ms": {n: round(x["avg_ms"], 4) for n, x in kern.items()},
        "roofline": roofline_of(w, wm, kern, peak),
        "data": "synthetic, drawn on the device (torch seeded generator; the recipe's distribution)",
    }
    log(f"{name}: {ms:.3f} ms per forward, " + ", ".join(f"{n} {x['avg_ms']:.3f}ms" for n, x in kern.items()))
    if args.dense_steps > 0:
        od = torch.empty_like(q)
        moba.dense(q, k, v, w.causal, out=od)  # one untimed run first
        torch.cuda.synchronize()
        td = time.perf_counter()
        moba.dense(q, k, v, w.causal, out=od)
        torch.cuda.synchronize()
        dense_ms = 1e3 * (time.perf_counter() - td)
        res["dense_causal"] = {"ms": round(dense_ms, 3), "speedup": round(dense_ms / ms, 2),
                               "tflops": round(wm["dense_flops"] / (dense_ms * 1e-3) / 1e12, 1), "timed_runs": 1}
        log(f"{name}: dense causal {dense_ms:.1f} ms, speedup {dense_ms / ms:.1f}x")
        del od
    del q, k, v
    torch.cuda.empty_cache()
    return res


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo) and the cores this
    process may run on."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return name, len(os.sched_getaffinity(0))


def cpu_baseline(w, n_rows):
    """The fp64 oracle on a bounded seeded sample of the workload, on this
    host's cores; extrapolated to a full forward (pool every head + every
    row) and reported as tokens/s."""
    from oracle import sampled
    rows = synth.sample_rows(w, n_rows)
    out = sampled.oracle_rows(w, rows)
    heads = out["heads"]
    pool_per_head = out["pool_s"] / heads
    row_s = (out["oracle_s"] - out["pool_s"]) / len(rows)
    bh = w.batch * w.heads
    cpu_seconds = pool_per_head * bh + row_s * bh * w.seq_len
    full_wall = cpu_seconds / out["workers"]
    model, affinity = cpu_model()
    return {
        "value": w.batch * w.seq_len / full_wall,
        "unit": "tokens/s",
        "cores": out["workers"],
        "kind": "oracle",
        "cpu_model": model,
        "affinity_cores": affinity,
        "near_ties": int(out["flag"].sum()),
        "sample": (f"{len(rows)} seeded query rows over {heads} heads of {w.name} (fp64 NumPy, "
                   f"{out['workers']} processes, 1 BLAS thread each, on {model}; {affinity} cores in this "
                   f"process's affinity, of which one GPU's host share is 16); measured {out['oracle_s']:.1f} CPU-s "
                   f"(pool {out['pool_s']:.1f} s + rows); value extrapolated to a full forward "
                   f"({bh} heads x {w.seq_len} rows) = {full_wall:.1f} s wall"),
    }


def measure_backward(w, wm, q, k, v, moba, torch, steps, warmup):
    """Timed moba_backward passes over the workload (the forward's o,
    block_idx and log-sum-exp resident in HBM, a seeded upstream gradient).
    Algorithmic work: 10*D flops per (query, attended key), the five
    D-length products of a softmax-attention backward (scores, dP, dQ, dK,
    dV); the kernels recompute the scores once more per pass."""
    o, idx, lse = moba.forward(q, k, v, w.block_size, w.top_k, w.causal, pooling=w.pooling,
                               gate_shared=w.gate_shared, return_lse=True)
    g = torch.Generator(device="cuda").manual_seed(w.seed + 1000)
    dout = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    torch.cuda.synchronize()

    def bstep():
        moba.backward(q, k, v, o, dout, idx, lse, w.block_size, w.top_k, w.causal)

    for _ in range(warmup):
        bstep()
    torch.cuda.synchronize()
    with moba.timing() as tm:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            bstep()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    del o, idx, lse, dout
    ms = 1e3 * elapsed / steps
    kern = {n: {"launches": c, "avg_ms": tot / c} for n, c, tot in tm.rows}
    D = w.head_dim
    past_keys = wm["past_flops"] // (4 * D)
    own_keys = wm["own_flops"] // (4 * D)
    flops = 10 * D * (past_keys + own_keys)
    # per-kernel algorithmic work: dq kernels 6*D per pair (scores, dP, dQ);
    # the dV pass 4*D (scores, dV), the dK pass 6*D (scores, dP, dK).
    units = {"bwd_dq_past": 6 * D * past_keys, "bwd_dq_own": 6 * D * own_keys,
             "bwd_dv": 4 * D * (past_keys + own_keys), "bwd_dk": 6 * D * (past_keys + own_keys)}
    dom = max((n for n in kern if n in units), key=lambda n: kern[n]["avg_ms"])
    ach = units[dom] / (kern[dom]["avg_ms"] * 1e-3) / 1e12
    return {
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
        "tokens_per_s": round(w.batch * w.seq_len / (ms * 1e-3), 1),
        "effective_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "pct_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {n: round(x["avg_ms"], 4) for n, x in kern.items()},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "work_per_launch": units[dom], "work_unit": "flop",
                     "avg_launch_ms": round(kern[dom]["avg_ms"], 4)},
    }


def backward_bench(args, w, wm, q, k, v, moba, torch):
    """--backward: one step = one moba_backward over the workload; its own
    JSON line (see measure_backward)."""
    if w.dtype != "bf16":
        print("the backward is built for bf16 workloads only", file=sys.stderr)
        sys.exit(2)
    log(f"backward: warmup {args.warmup}, timing {args.steps} steps")
    r = measure_backward(w, wm, q, k, v, moba, torch, args.steps, args.warmup)
    log("kernels: " + ", ".join(f"{n} {x:.3f}ms" for n, x in r["kernels_ms"].items()))
    D = w.head_dim
    line = {
        "metric": "MoBA bwd tokens/sec + effective TFLOP/s (% bf16 MFMA peak)",
        "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (the forward's recipe; upstream gradient ~ N(0,1))",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "kv_heads": w.kvh, "seq_len": w.seq_len,
                   "head_dim": D, "block_size": w.block_size, "top_k": w.top_k, "causal": w.causal,
                   "parallelism": "single GPU"},
        "effective_tflops": r["effective_tflops"], "pct_peak": r["pct_peak"], "kernels_ms": r["kernels_ms"],
        "roofline": r["roofline"], "cpu_baseline": None,
    }
    if args.cpu_rows > 0:
        from oracle import sampled
        n = min(args.cpu_rows, 16384)
        log(f"cpu baseline: oracle backward on {n} sampled rows")
        rows = synth.sample_rows(w, n)
        pool_s, row_s, nrows, heads, workers = sampled.oracle_backward_rows(w, rows)
        cpu_s = pool_s + row_s
        bh = w.batch * w.heads
        full_wall = (pool_s / heads * bh + row_s / nrows * bh * w.seq_len) / workers
        line["cpu_baseline"] = {
            "value": w.batch * w.seq_len / full_wall, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": (f"{nrows} seeded query rows over {heads} heads of {w.name}: routing plus the fp64 "
                       f"softmax-attention gradient of each row (NumPy, {workers} processes, 1 BLAS thread each); "
                       f"measured {cpu_s:.1f} CPU-s (pooling {pool_s:.1f} s + rows); value extrapolated to every head "
                       f"and row ({bh} heads x {w.seq_len}) "
                       f"= {full_wall:.1f} s wall"),
        }
        log(f"cpu baseline: {line['cpu_baseline']['value']:.1f} tokens/s on {workers} cores")
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline_32k", choices=synth.WORKLOAD_ORDER + synth.POOLING_VARIANTS + synth.SHAPE_VARIANTS
                    + synth.GQA_VARIANTS)
    ap.add_argument("--dense-steps", type=int, default=2, help="timed dense causal forwards (0 = skip)")
    ap.add_argument("--cpu-rows", type=int, default=65536, help="oracle sample size (0 = skip)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a plain device copy whose "
                         "HBM counters calibrate FETCH_SIZE/WRITE_SIZE readings)")
    ap.add_argument("--backward", action="store_true",
                    help="time the MoBA backward (dq, dk, dv for a fixed block choice) instead of the forward "
                         "and print its own JSON line (bf16 workloads)")
    ap.add_argument("--device-inputs", action="store_true",
                    help="draw the workload's inputs on the device (the recipe's distribution, torch's seeded "
                         "generator) instead of the seeded host streams: for profiling the long workloads, whose "
                         "host streams take minutes to generate")
    ap.add_argument("--long", default="long_128k,long_1m",
                    help="comma-separated long-context workloads measured as sub-results of the main line "
                         "('' = none)")
    ap.add_argument("--long-steps", type=int, default=3, help="timed forwards per long-context sub-result")
    ap.add_argument("--backward-steps", type=int, default=5,
                    help="timed moba_backward passes reported as the line's backward sub-result (0 = skip)")
    ap.add_argument("--gen-workers", type=int, default=None,
                    help="processes generating the inputs (default: one per core, up to 16; use 1 under a profiler)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(MoBA shards over heads with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_long_context_moba_amd as moba

    w = synth.WORKLOADS[args.workload]
    wm = work_model(w)
    log(f"workload {w.name}: B={w.batch} H={w.heads} S={w.seq_len} D={w.head_dim} "
        f"block={w.block_size} top_k={w.top_k} {w.dtype}; generating inputs")
    t0 = time.time()
    q, k, v = upload_device(w, torch, 1000 + w.seed) if args.device_inputs else upload(w, torch, args.gen_workers)
    log(f"inputs resident in HBM after {time.time() - t0:.1f}s")
    p = moba.problem(q, w.block_size, w.top_k, w.causal, w.pooling, w.kvh, w.gate_shared)
    ws = torch.empty(moba.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    idx = torch.empty((w.batch, w.heads, w.seq_len, w.top_k), dtype=torch.int32, device="cuda")

    def step():
        moba.forward(q, k, v, w.block_size, w.top_k, w.causal, out=o, idx=idx, workspace=ws, pooling=w.pooling,
                     gate_shared=w.gate_shared)

    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")
        del src, dst
    if args.backward:
        return backward_bench(args, w, wm, q, k, v, moba, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")
    with moba.timing() as tm:
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
    ms_per_step = 1e3 * elapsed / args.steps
    kern = {name: {"launches": n, "avg_ms": tot / n, "total_ms": tot} for name, n, tot in tm.rows}
    log("kernels: " + ", ".join(f"{n} {v['avg_ms']:.3f}ms" for n, v in kern.items()))

    algo_flops = wm["gate_flops"] + wm["past_flops"] + wm["own_flops"]
    eff_tflops = algo_flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS

    units = kernel_units(w, wm)
    dom = max((n for n in kern if n in units), key=lambda n: kern[n]["total_ms"])
    bound, work, unit = units[dom]
    avg_s = kern[dom]["avg_ms"] * 1e-3
    if bound == "hbm":
        achieved, rpeak, runit = work / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, rpeak, runit = work / avg_s / 1e12, peak, "TFLOP/s"
    roofline = {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": rpeak, "unit": runit,
                "frac": round(achieved / rpeak, 4), "traffic": measured_traffic(dom, w.name),
                "work_per_launch": work, "work_unit": unit, "avg_launch_ms": round(kern[dom]["avg_ms"], 4)}
    pool_hbm = None
    if "pool" in kern and "pool" in units:
        gbs = units["pool"][1] / (kern["pool"]["avg_ms"] * 1e-3) / 1e9
        pool_hbm = {"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    attn_gate_ms = sum(kern[n]["avg_ms"] for n in ("gate_topk", "gather_attn", "diag_merge") if n in kern)
    attn_gate_frac = (wm["gate_flops"] + wm["past_flops"] + wm["own_flops"]) / (attn_gate_ms * 1e-3) / 1e12 / peak

    dense = None
    if args.dense_steps > 0:
        od = torch.empty_like(q)
        moba.dense(q, k, v, w.causal, out=od)
        torch.cuda.synchronize()
        td = time.perf_counter()
        for _ in range(args.dense_steps):
            moba.dense(q, k, v, w.causal, out=od)
        torch.cuda.synchronize()
        dense_ms = 1e3 * (time.perf_counter() - td) / args.dense_steps
        dense = {"ms": round(dense_ms, 3), "speedup": round(dense_ms / ms_per_step, 2),
                 "tflops": round(wm["dense_flops"] / (dense_ms * 1e-3) / 1e12, 1)}
        log(f"dense causal: {dense_ms:.3f} ms, speedup {dense['speedup']}x")
        del od

    cpu = None
    if args.cpu_rows > 0:
        log(f"cpu baseline: oracle on {args.cpu_rows} sampled rows")
        cpu = cpu_baseline(w, args.cpu_rows)
        log(f"cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} cores")

    backward = None
    if args.backward_steps > 0 and w.dtype == "bf16" and w.seq_len % 64 == 0:
        log(f"backward: timing {args.backward_steps} passes")
        backward = measure_backward(w, wm, q, k, v, moba, torch, args.backward_steps, 2)
        log(f"backward: {backward['ms_per_step']} ms ({backward['pct_peak']} % of peak)")

    long_results = []
    names = [n for n in args.long.split(",") if n and n != w.name]
    if names:
        del q, k, v, o, idx, ws
        torch.cuda.empty_cache()
        for name in names:
            long_results.append(long_context_result(name, args, moba, torch))

    tokens = w.batch * w.seq_len
    line = {
        "metric": METRIC,
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded q, v ~ N(0,1); k ~ N(0,1) + per-block N(0, 0.5^2) bias)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                   "head_dim": w.head_dim, "block_size": w.block_size, "top_k": w.top_k,
                   "causal": w.causal, "pooling": w.pooling, "kv_heads": w.kvh, "gate_shared": w.gate_shared,
                   "parallelism": "single GPU"},
        "effective_tflops": round(eff_tflops, 2),
        "pct_peak": round(100 * eff_tflops / peak, 2),
        "attn_gate_kernels_pct_peak": round(100 * attn_gate_frac, 2),
        "sparsity": {"realized": round(1 - wm["attended_keys"] / wm["dense_keys"], 4),
                     "theoretical_1_minus_k_over_nb": round(1 - w.top_k / w.n_blocks, 4)},
        "kernels_ms": {n: round(v["avg_ms"], 4) for n, v in kern.items()},
        "pool_hbm": pool_hbm,
        "dense_causal": dense,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "backward": backward,
        "long_context": long_results,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
