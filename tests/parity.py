"""Parity helpers shared by the GPU tests: run the HIP path through the C ABI
binding, run the fp64 oracle on the same seeded inputs, and compare.

Acceptance (per query row):
  * idx must equal the oracle's exactly unless the oracle flags the row as a
    near-tie (its last kept and first dropped scores within 1e-5 relative);
  * a flagged row may break the tie either way: the GPU set must hold the
    own block, every eligible block scoring above a + tau and only eligible
    blocks scoring at least b - tau (tau = 1e-5 * max(|a|, |b|)); its output
    is then compared with the oracle attending the GPU's own choice;
  * max |o_gpu - o_oracle| <= 1e-4 (fp32) or 2e-2 (bf16).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moba as orc

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def check_rows(gpu_o, gpu_idx, res, rows_t, q, k, v, block_size, top_k, causal, dtype, label="", q_gate=None):
    """Compare GPU rows (o [R, D], idx [R, top_k]) of one head with the
    oracle's forward_head result `res` for the same rows. Returns stats.
    q_gate: the query the gate scores with, if not q (a shared gate scores
    the group's summed query)."""
    q_gate = q if q_gate is None else q_gate
    tol = TOL[dtype]
    kbar = res["kbar"]
    n_flag = n_tie_diff = 0
    max_err = 0.0
    sq = 0.0
    for r, t in enumerate(rows_t):
        t = int(t)
        c = t // block_size
        gi = [int(x) for x in gpu_idx[r]]
        oi = [int(x) for x in res["idx"][r]]
        ref = res["o"][r]
        if gi != oi:
            assert res["flag"][r], f"{label} t={t}: idx {gi} != oracle {oi} (not a near-tie)"
            n_tie_diff += 1
            a, b = res["a"][r], res["b"][r]
            tau = orc.NEAR_TIE_REL * max(abs(a), abs(b))
            elig = set(int(j) for j in orc.eligible_blocks(c, kbar.shape[0], causal))
            s = {j: float(kbar[j] @ np.asarray(q_gate[t], np.float64)) for j in elig}
            chosen = set(j for j in gi if j >= 0)
            assert c in chosen, f"{label} t={t}: own block missing"
            assert all(s[j] <= a + tau or j in chosen for j in elig), f"{label} t={t}: dropped a clear winner"
            assert all(j == c or (j in elig and s[j] >= b - tau) for j in chosen), f"{label} t={t}: bad pick"
            assert len(chosen) == len([x for x in oi if x >= 0])
            ref = orc.attend_with_idx(q[t], k, v, t, np.array(gi), block_size, causal)
        n_flag += bool(res["flag"][r])
        err = np.abs(gpu_o[r].astype(np.float64) - ref).max()
        sq += float(((gpu_o[r].astype(np.float64) - ref) ** 2).mean())
        max_err = max(max_err, err)
        assert err <= tol, f"{label} t={t}: max|o - oracle| = {err:.3e} > {tol}"
    return {"rows": len(rows_t), "max_err": max_err, "rms": (sq / max(1, len(rows_t))) ** 0.5,
            "flagged": n_flag, "tie_diff": n_tie_diff}
