"""GPU parity of the MoBA backward (bf16) against the fp64 oracle's
backward_head, every row and every key, with the GPU forward's block
choice held fixed on both sides (the gradient is defined for a given
choice). Also the forward's log-sum-exp output against the oracle's."""
import numpy as np
import pytest
import torch

from oracle import moba as orc
from tests.parity import say, to_dev

pytestmark = pytest.mark.gpu

# Tolerances (bf16 inputs, fp32 accumulation, P and dS rounded to bf16 for
# the MFMA products, as P is in the forward): the error of a gradient entry
# is a sum of per-key terms each off by about 2^-8 of its size, so it is
# bounded relative to the tensor's own scale: max |err| <= 2e-2 * max |ref|.
REL = 2e-2
LSE_TOL = 1e-4  # fp32 log-sum-exp of logits of size ~10: rounding ~1e-6
# Scale floor: a query whose only key is itself has no gradient (a one-key
# softmax), so a reference can be exactly zero; the GPU then holds the
# rounding of delta - dP (about 1e-7), judged against this floor.
SCALE_FLOOR = 1e-3


def _round(x):
    import synth
    return synth.round_to_bf16(x)


def _inputs(seed, B, H, Hkv, S, D, Bs, bias=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, S, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    nb = -(-S // Bs)
    k += np.repeat(rng.normal(0, bias, (B, Hkv, nb, D)).astype(np.float32), Bs, axis=2)[:, :, :S]
    v = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    do = rng.standard_normal((B, H, S, D)).astype(np.float32)
    return _round(q), _round(k), _round(v), _round(do)


CASES = [
    # label, seed, B, H, Hkv, S, D, Bs, top_k, causal, shared
    ("d128-bs128-k3", 70, 1, 2, 2, 1024, 128, 128, 3, True, False),
    ("d64-bs64-k4-noncausal", 71, 1, 2, 2, 512, 64, 64, 4, False, False),
    ("d128-bs256-short192", 72, 1, 2, 2, 1216, 128, 256, 3, True, False),
    ("d128-k1", 73, 1, 1, 1, 512, 128, 128, 1, True, False),
    ("d64-topk-all", 74, 1, 1, 1, 512, 64, 64, 9, True, False),
    ("d128-gqa2-shared", 75, 1, 4, 2, 1024, 128, 128, 3, True, True),
    ("d128-gqa4-per-head-b2", 76, 2, 4, 1, 512, 128, 128, 2, True, False),
    # any length: partial last query tiles and key subtiles
    ("d128-bs128-len1000", 77, 1, 2, 2, 1000, 128, 128, 3, True, False),
    ("d64-bs64-len77-noncausal", 78, 1, 2, 2, 77, 64, 64, 3, False, False),
    ("d128-bs256-len1000-noncausal", 79, 1, 2, 2, 1000, 128, 256, 3, False, False),
    ("d128-gqa2-shared-len513-b2", 84, 2, 4, 2, 513, 128, 64, 4, True, True),
    ("d128-len1", 85, 1, 2, 2, 1, 128, 64, 3, True, False),
    ("d64-bs64-len65-noncausal", 86, 1, 1, 1, 65, 64, 64, 2, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(case):
    import sparse_long_context_moba_amd as moba
    label, seed, B, H, Hkv, S, D, Bs, top_k, causal, shared = case
    q, k, v, do = _inputs(seed, B, H, Hkv, S, D, Bs)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    say(f"[gpu] backward {label}: q={q.shape} kv={k.shape} Bs={Bs} top_k={top_k} causal={causal} shared={shared}")
    o, idx, lse = moba.forward(qd, kd, vd, Bs, top_k, causal, gate_shared=shared, return_lse=True)
    dq, dk, dv = moba.backward(qd, kd, vd, o, dod, idx, lse, Bs, top_k, causal)
    dq2, dk2, dv2 = moba.backward(qd, kd, vd, o, dod, idx, lse, Bs, top_k, causal)
    torch.cuda.synchronize()
    for x, y in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), "backward is not run-to-run bit-identical"
    _check_against_oracle(label, q, k, v, do, idx, lse, dq, dk, dv, Bs, causal)


def _check_against_oracle(label, q, k, v, do, idx, lse, dq, dk, dv, Bs, causal):
    """Every dq row and lse value per query head, and dk, dv per key/value
    head (the oracle's per-head gradients summed over the heads that read
    it), against backward_head with the GPU's block choice."""
    idx = idx.cpu().numpy()
    lse = lse.cpu().numpy()
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0, "lse": 0.0}
    for b in range(B):
        for hk in range(Hkv):
            rdk = np.zeros((S, D))
            rdv = np.zeros((S, D))
            for g in range(G):
                h = hk * G + g
                gq, gk, gv, glse = orc.backward_head(q[b, h], k[b, hk], v[b, hk], do[b, h], idx[b, h], Bs, causal)
                rdk += gk
                rdv += gv
                e_lse = np.abs(lse[b, h] - glse).max()
                assert e_lse <= LSE_TOL, f"{label} b={b} h={h}: lse error {e_lse:.3e}"
                e = np.abs(dq[b, h] - gq).max()
                sc = max(np.abs(gq).max(), SCALE_FLOOR)
                assert e <= REL * sc, f"{label} b={b} h={h}: dq error {e:.3e} (scale {np.abs(gq).max():.3e})"
                worst["dq"] = max(worst["dq"], e / sc)
                worst["lse"] = max(worst["lse"], e_lse)
            for name, got, ref in (("dk", dk[b, hk], rdk), ("dv", dv[b, hk], rdv)):
                e = np.abs(got - ref).max()
                sc = max(np.abs(ref).max(), SCALE_FLOOR)
                assert e <= REL * sc, f"{label} b={b} kv={hk}: {name} error {e:.3e} (scale {np.abs(ref).max():.3e})"
                worst[name] = max(worst[name], e / sc)
    say(f"[gpu] backward {label}: ok, max error / scale: " + ", ".join(f"{n}={v:.2e}" for n, v in worst.items()))


VARLEN_CASES = [
    # label, seed, H, Hkv, D, Bs, top_k, causal, shared, lengths
    ("d128-bs128-causal", 80, 2, 2, 128, 128, 3, True, False, [576, 1024, 192]),
    ("d64-bs64-noncausal-gqa2-shared", 81, 4, 2, 64, 64, 3, False, True, [128, 704, 64]),
    ("d128-bs128-causal-ragged", 82, 2, 2, 128, 128, 3, True, False, [1000, 77, 513]),
    ("d64-bs64-noncausal-with-1-token", 83, 2, 2, 64, 64, 3, False, False, [1, 200, 64]),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[c[0] for c in VARLEN_CASES])
def test_backward_varlen(case):
    """The backward of a varlen batch (forward_varlen with its log-sum-exp,
    then backward_varlen): every sequence's lse, dq, dk and dv bit-identical
    to those of that sequence run alone, and the first sequence's against
    the oracle."""
    import sparse_long_context_moba_amd as moba
    label, seed, H, Hkv, D, Bs, top_k, causal, shared, lengths = case
    seqs = [_inputs(seed + i, 1, H, Hkv, n, D, Bs) for i, n in enumerate(lengths)]
    dev = [[to_dev(x, "bf16") for x in s] for s in seqs]
    qp, cu = moba.pack_varlen([d[0] for d in dev])
    kp, _ = moba.pack_varlen([d[1] for d in dev])
    vp, _ = moba.pack_varlen([d[2] for d in dev])
    dop, _ = moba.pack_varlen([d[3] for d in dev])
    say(f"[gpu] backward varlen {label}: lengths={lengths} cu={cu}")
    o, idx, lse = moba.forward_varlen(qp, kp, vp, cu, H, Bs, top_k, causal, kv_heads=Hkv, gate_shared=shared,
                                      return_lse=True)
    dq, dk, dv = moba.backward_varlen(qp, kp, vp, o, dop, idx, lse, cu, H, Bs, top_k, causal, kv_heads=Hkv,
                                      gate_shared=shared)
    torch.cuda.synchronize()
    parts = {"dq": moba.unpack_varlen(dq, cu, H), "dk": moba.unpack_varlen(dk, cu, Hkv),
             "dv": moba.unpack_varlen(dv, cu, Hkv)}
    idxs = moba.unpack_varlen(idx, cu, H)
    for i, d in enumerate(dev):
        n = lengths[i]
        lse_i = lse[cu[i] * H:cu[i + 1] * H].view(1, H, n)
        o1, i1, l1 = moba.forward(d[0], d[1], d[2], Bs, top_k, causal, gate_shared=shared, return_lse=True)
        assert torch.equal(idxs[i], i1), f"sequence {i}: block choice differs from the sequence alone"
        assert torch.equal(lse_i.view(torch.int32), l1.view(torch.int32)), f"sequence {i}: lse differs"
        g1 = moba.backward(d[0], d[1], d[2], o1, d[3], i1, l1, Bs, top_k, causal)
        torch.cuda.synchronize()
        for name, ref in zip(("dq", "dk", "dv"), g1):
            got = parts[name][i].contiguous()
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"sequence {i}: {name} differs"
        if i == 0:
            q, k, v, do = seqs[0]
            _check_against_oracle(f"{label} seq=0", q, k, v, do, i1, l1, g1[0], g1[1], g1[2], Bs, causal)
    say(f"[gpu] backward varlen {label}: ok")


def _check_sampled(w):
    """dq on 256 seeded sampled rows (plus edge rows), and dk, dv on every
    key of two blocks (the first and the last) of the first and the last
    head, each summed by the oracle over every query that attends those
    keys."""
    import synth
    import sparse_long_context_moba_amd as moba
    S, D, Bs = w.seq_len, w.head_dim, w.block_size
    say(f"[gpu] backward {w.name}: generating inputs")
    q = torch.empty((1, w.heads, S, D), dtype=torch.bfloat16, device="cuda")
    k, v = (torch.empty_like(q) for _ in range(2))
    host = {}
    for b, hk, qh, kh, vh in synth.iter_groups_parallel(w):
        for dst, x in ((q, qh), (k, kh[None]), (v, vh[None])):
            dst[b, hk:hk + 1].copy_(torch.from_numpy(x).view(torch.bfloat16))
        host[hk] = tuple((x.view(np.uint16).astype(np.uint32) << 16).view(np.float32) for x in (qh[0], kh, vh))
    g = torch.Generator(device="cuda").manual_seed(w.seed + 1000)
    dout = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    o, idx, lse = moba.forward(q, k, v, Bs, w.top_k, w.causal, return_lse=True)
    dq, dk, dv = moba.backward(q, k, v, o, dout, idx, lse, Bs, w.top_k, w.causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for h in (0, w.heads - 1):
        qh, kh, vh = host[h]
        doh = dout[0, h].float().cpu().numpy()
        ih = idx[0, h].cpu().numpy()
        dqh, dkh, dvh = (x[0, h].float().cpu().numpy() for x in (dq, dk, dv))
        rows = np.unique(np.concatenate([rng.choice(S, 256, replace=False), [0, Bs - 1, Bs, S - 1]]))
        ref = np.stack([orc.attend_grad(qh[t], kh, vh, orc.attended_keys(int(t), ih[t], Bs, True, S), doh[t])[0]
                        for t in rows])
        e = np.abs(dqh[rows] - ref).max()
        assert e <= REL * np.abs(ref).max(), f"h={h}: dq error {e:.3e} (scale {np.abs(ref).max():.3e})"
        for j in (0, S // Bs - 1):
            lo, hi = j * Bs, (j + 1) * Bs
            users = np.nonzero((ih == j).any(axis=1))[0]
            rdk = np.zeros((Bs, D))
            rdv = np.zeros((Bs, D))
            for t in users:
                keys = orc.attended_keys(int(t), ih[t], Bs, True, S)
                _, gk, gv = orc.attend_grad(qh[t], kh, vh, keys, doh[t])
                sel = (keys >= lo) & (keys < hi)
                rdk[keys[sel] - lo] += gk[sel]
                rdv[keys[sel] - lo] += gv[sel]
            for name, got, r in (("dk", dkh[lo:hi], rdk), ("dv", dvh[lo:hi], rdv)):
                e = np.abs(got - r).max()
                assert e <= REL * np.abs(r).max(), f"h={h} block={j}: {name} error {e:.3e} (scale {np.abs(r).max():.3e})"
            say(f"[gpu] backward {w.name} h={h} block={j}: {len(users)} queries attend it; ok")


def test_backward_headline_sampled():
    """headline_32k (32 heads, 32768 tokens, block 512, top_k 3) at full
    size, in the launch configuration bench.py --backward times."""
    import synth
    _check_sampled(synth.WORKLOADS["headline_32k"])


def test_backward_64k_two_heads_sampled():
    """65536 tokens, 2 heads, block 512, top_k 3: past 32768 tokens the
    ordered ranks of the backward's lists take 1024-query chunks (256 up to
    that length), so this covers the other chunk size."""
    import synth
    _check_sampled(synth.Workload("bwd_64k_2h", 1, 2, 65536, 128, 512, 3, True, "bf16", 21))


def _edit_rows(idx, Bs):
    """block_idx rows rewritten with entries the backward must skip (out of
    range, negative after the valid ones, the own block repeated, future
    blocks, a fourth past block beyond the cap) and the valid past blocks
    reordered, so that the blocks the backward keeps are exactly the
    original ones. idx: int [S, 4] of one head, causal, top_k 4."""
    out = idx.copy()
    S = idx.shape[0]
    for t in range(S):
        c = t // Bs
        row = [int(j) for j in idx[t] if j >= 0]
        past = [j for j in row if j != c]
        if c == 0:
            out[t] = [0, 7, 5, 99]
        elif c == 1:
            out[t] = [1, 0, 1, 4000]
        elif c == 2:
            out[t] = [2, past[1], past[0], -3]
        elif t % 2 == 0 or c == 3:
            out[t] = [c, past[2], past[0], past[1]]
        else:
            extra = next(j for j in range(c) if j not in past)
            out[t] = [past[0], past[1], past[2], extra]
    return out


def _kept_past_blocks(row, c, n_blocks, k_eff, causal=True):
    """The documented reading of a row: up to the first -1, skip entries that
    name no past block the query may attend, keep the first
    min(k_eff - 1, eligible) of the rest."""
    cap = min(k_eff - 1, c if causal else n_blocks - 1)
    kept = []
    for j in row:
        if j < 0 or len(kept) >= cap:
            break
        if j < n_blocks and j != c and (not causal or j < c):
            kept.append(int(j))
    return kept


def test_backward_skips_entries_that_name_no_past_block():
    """A block_idx edited by the caller: entries that name no past block the
    query may attend are skipped and at most min(top_k, n_blocks) - 1 past
    blocks per row are used, in the same way by every kernel that reads the
    rows. With edits that keep the same past blocks, the gradients equal
    the oracle's for the forward's own choice."""
    import sparse_long_context_moba_amd as moba
    B, H, S, D, Bs, top_k = 1, 2, 2048, 128, 256, 4
    q, k, v, do = _inputs(77, B, H, H, S, D, Bs)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    o, idx, lse = moba.forward(qd, kd, vd, Bs, top_k, True, return_lse=True)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    edited = np.stack([_edit_rows(idx_h[0, h], Bs) for h in range(H)])[None].astype(np.int32)
    nb = S // Bs
    for h in range(H):
        for t in range(S):
            c = t // Bs
            orig = sorted(j for j in idx_h[0, h, t] if 0 <= j != c)
            assert sorted(_kept_past_blocks(edited[0, h, t], c, nb, top_k)) == orig, (h, t)
    say(f"[gpu] backward with edited block_idx rows: S={S} Bs={Bs} top_k={top_k}")
    dq, dk, dv = moba.backward(qd, kd, vd, o, dod, torch.from_numpy(edited).cuda(), lse, Bs, top_k, True)
    torch.cuda.synchronize()
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    for h in range(H):
        gq, gk, gv, _ = orc.backward_head(q[0, h], k[0, h], v[0, h], do[0, h], idx_h[0, h], Bs, True)
        for name, got, ref in (("dq", dq[0, h], gq), ("dk", dk[0, h], gk), ("dv", dv[0, h], gv)):
            e = np.abs(got - ref).max()
            assert e <= REL * np.abs(ref).max(), f"h={h}: {name} error {e:.3e} (scale {np.abs(ref).max():.3e})"
    say("[gpu] backward with edited rows: ok")
