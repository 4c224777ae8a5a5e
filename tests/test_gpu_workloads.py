"""GPU parity at the named workloads' full sizes, in the launch
configuration bench.py times: the whole forward runs on the GPU, and 4096
seeded sampled query rows (plus edge rows) are checked against the fp64
oracle on the same seeded inputs."""
import time

import numpy as np
import pytest
import torch

import synth
from oracle import moba as orc
from tests.parity import check_rows, say

pytestmark = pytest.mark.gpu


def _upload(w):
    """Generate the workload's inputs per key/value head and its group of
    query heads on the host (worker processes) and copy them into device
    tensors; keep the host copies for the oracle, keyed by (b, kv head)."""
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    G = w.group
    qd = torch.empty((w.batch, w.heads, w.seq_len, w.head_dim), dtype=tdt, device="cuda")
    kd, vd = (torch.empty((w.batch, w.kvh, w.seq_len, w.head_dim), dtype=tdt, device="cuda") for _ in range(2))
    host = {}
    cast = (lambda t: t.view(torch.bfloat16)) if w.dtype == "bf16" else (lambda t: t)
    for b, hk, q, k, v in synth.iter_groups_parallel(w):
        qd[b, hk * G:(hk + 1) * G].copy_(cast(torch.from_numpy(q)))
        kd[b, hk].copy_(cast(torch.from_numpy(k)))
        vd[b, hk].copy_(cast(torch.from_numpy(v)))
        host[(b, hk)] = (q, k, v)
    return (qd, kd, vd), host


def _as_f32(x, dtype):
    if dtype == "bf16":
        return (x.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return x


def _oracle_head(args):
    """Oracle rows of query head g of a group (all G heads' queries given)."""
    qb, kb, vb, g, rows, w = args
    qs, k, v = (_as_f32(x, w.dtype) for x in (qb, kb, vb))
    if w.gate_shared:
        res = orc.forward_group(qs, k, v, w.block_size, w.top_k, w.causal, rows=rows, pooling=w.pooling,
                                shared_gate=True)[g]
        q_gate = qs.astype(np.float64).sum(axis=0)
    else:
        res = orc.forward_head(qs[g], k, v, w.block_size, w.top_k, w.causal, rows=rows, pooling=w.pooling)
        q_gate = None
    return res, qs[g], k, v, q_gate


def _run(name, n_rows=4096):
    import sparse_long_context_moba_amd as moba
    w = synth.WORKLOADS[name]
    t0 = time.time()
    say(f"[gpu] {name}: generating and uploading inputs")
    (qd, kd, vd), host = _upload(w)
    say(f"[gpu] {name}: inputs ready in {time.time() - t0:.1f}s; running moba.forward")
    kw = dict(pooling=w.pooling, gate_shared=w.gate_shared)
    o, idx = moba.forward(qd, kd, vd, w.block_size, w.top_k, w.causal, **kw)
    torch.cuda.synchronize()
    # Run-to-run: every output bit and index must repeat (the path has no
    # floating-point atomics, so any difference is a race).
    o2, idx2 = moba.forward(qd, kd, vd, w.block_size, w.top_k, w.causal, **kw)
    torch.cuda.synchronize()
    bits = torch.int16 if o.dtype == torch.bfloat16 else torch.int32
    n_diff = int((o.view(bits) != o2.view(bits)).sum().item())
    assert n_diff == 0 and torch.equal(idx, idx2), f"{name}: {n_diff} output values differ between two runs"
    del o2, idx2
    rows = synth.sample_rows(w, n_rows)
    sel = torch.from_numpy(rows).cuda()
    o_rows = o[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    idx_rows = idx[sel[:, 0], sel[:, 1], sel[:, 2]].cpu().numpy()
    del o, idx, qd, kd, vd
    torch.cuda.empty_cache()
    say(f"[gpu] {name}: forward done; oracle on {len(rows)} rows")
    groups = {}
    for i, (b, h, t) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append(i)
    stats = {"rows": 0, "max_err": 0.0, "flagged": 0, "tie_diff": 0}
    import multiprocessing as mp
    keys = sorted(groups)
    G = w.group
    jobs = [(*host[(bh[0], bh[1] // G)], bh[1] % G, rows[groups[bh], 2], w) for bh in keys]
    with mp.get_context("fork").Pool(min(16, len(jobs))) as pool:
        for bh, (res, q, k, v, q_gate) in zip(keys, pool.imap(_oracle_head, jobs)):
            ii = groups[bh]
            st = check_rows(o_rows[ii], idx_rows[ii], res, rows[ii, 2], q, k, v, w.block_size,
                            w.top_k, w.causal, w.dtype, label=f"{name} b={bh[0]} h={bh[1]}", q_gate=q_gate)
            stats["rows"] += st["rows"]
            stats["max_err"] = max(stats["max_err"], st["max_err"])
            stats["flagged"] += st["flagged"]
            stats["tie_diff"] += st["tie_diff"]
    say(f"[gpu] {name}: ok {stats} in {time.time() - t0:.1f}s")
    assert stats["rows"] == len(rows)


def _oracle_dense_rows(args):
    qb, kb, vb, rows, dtype, causal = args
    q, k, v = (_as_f32(x, dtype) for x in (qb, kb, vb))
    return orc.dense_attention(q, k, v, causal, rows=rows)


def _run_dense(name, n_rows=4096):
    """The dense kernel (the speedup's denominator) at a workload's full
    size, in the launch bench.py times: sampled rows against the oracle's
    plain softmax attention."""
    import sparse_long_context_moba_amd as moba
    w = synth.WORKLOADS[name]
    t0 = time.time()
    say(f"[gpu] dense {name}: generating and uploading inputs")
    (qd, kd, vd), host = _upload(w)
    say(f"[gpu] dense {name}: inputs ready in {time.time() - t0:.1f}s; running moba.dense")
    o = moba.dense(qd, kd, vd, w.causal)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w, n_rows)
    sel = torch.from_numpy(rows).cuda()
    o_rows = o[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    del o, qd, kd, vd
    torch.cuda.empty_cache()
    say(f"[gpu] dense {name}: done; oracle on {len(rows)} rows")
    groups = {}
    for i, (b, h, t) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append(i)
    keys = sorted(groups)
    G = w.group
    jobs = []
    for b, h in keys:
        qg, kh, vh = host[(b, h // G)]
        jobs.append((qg[h % G], kh, vh, rows[groups[(b, h)], 2], w.dtype, w.causal))
    import multiprocessing as mp
    worst = 0.0
    tol = 2e-2 if w.dtype == "bf16" else 1e-4
    with mp.get_context("fork").Pool(min(16, len(jobs))) as pool:
        for bh, ref in zip(keys, pool.imap(_oracle_dense_rows, jobs)):
            ii = groups[bh]
            err = np.abs(o_rows[ii].astype(np.float64) - ref).max(axis=1)
            worst = max(worst, float(err.max()))
            bad = np.nonzero(err > tol)[0]
            assert len(bad) == 0, (f"dense {name} b={bh[0]} h={bh[1]} t={rows[ii][bad[0], 2]}: "
                                   f"max|o - oracle| = {err[bad[0]]:.3e} > {tol}")
    say(f"[gpu] dense {name}: ok, {len(rows)} rows, max_err={worst:.3e} in {time.time() - t0:.1f}s")


def test_dense_headline_32k_sampled():
    _run_dense("headline_32k")


def test_tiny_all_rows():
    _run("tiny", n_rows=4096)


def test_headline_32k_sampled():
    _run("headline_32k")


def test_headline_32k_max_pooling_sampled():
    _run("headline_32k_max")


def test_headline_32k_meanmax_pooling_sampled():
    _run("headline_32k_meanmax")


def test_headline_short_last_block_sampled():
    _run("headline_33k_short_block")


def test_headline_gqa4_per_head_sampled():
    _run("headline_32k_gqa4")


def test_headline_gqa4_shared_gate_sampled():
    _run("headline_32k_gqa4_shared")


def test_coarse_32k_sampled():
    _run("coarse_32k")


def test_long_128k_sampled():
    _run("long_128k")


@pytest.mark.slow
def test_long_1m_sampled():
    _run("long_1m")
