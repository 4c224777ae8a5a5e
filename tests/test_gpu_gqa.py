"""GPU parity for grouped-query attention: several query heads read one
key/value head, each routing on its own or the group routing once on the
sum of its heads' gate scores. Every row is checked against the oracle's
forward_group (which is pinned on the CPU: per-head equality without
sharing, brute force over subsets on the summed score, and full attention
for top_k >= n_blocks)."""
import numpy as np
import pytest
import torch

from oracle import moba as orc
from tests.parity import check_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _round(x, dtype):
    import synth
    return synth.round_to_bf16(x) if dtype == "bf16" else x.astype(np.float32)


def _inputs(seed, B, H, Hkv, S, D, Bs, dtype, bias=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, S, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    nb = -(-S // Bs)
    k += np.repeat(rng.normal(0, bias, (B, Hkv, nb, D)).astype(np.float32), Bs, axis=2)[:, :, :S]
    v = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    return _round(q, dtype), _round(k, dtype), _round(v, dtype)


def _check(q, k, v, o, idx, Bs, top_k, causal, dtype, shared, label):
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    worst = 0.0
    for b in range(B):
        for hk in range(Hkv):
            qs = q[b, hk * G:(hk + 1) * G]
            outs = orc.forward_group(qs, k[b, hk], v[b, hk], Bs, top_k, causal, shared_gate=shared)
            q_gate = qs.astype(np.float64).sum(axis=0) if shared else None
            for g in range(G):
                h = hk * G + g
                st = check_rows(o[b, h], idx[b, h], outs[g], np.arange(S), q[b, h], k[b, hk], v[b, hk], Bs,
                                top_k, causal, dtype, label=f"{label} b={b} h={h}",
                                q_gate=q_gate if shared else q[b, h])
                worst = max(worst, st["max_err"])
            if shared:
                for g in range(1, G):
                    assert np.array_equal(idx[b, hk * G], idx[b, hk * G + g]), f"{label}: group {hk} split"
    return worst


CASES = [
    # label, seed, B, H, Hkv, S, D, Bs, top_k, causal, dtype, shared
    ("bf16-d128-g4-per-head", 40, 1, 4, 1, 1024, 128, 128, 3, True, "bf16", False),
    ("bf16-d128-g4-shared", 40, 1, 4, 1, 1024, 128, 128, 3, True, "bf16", True),
    ("bf16-d64-g2-shared-k5", 41, 2, 4, 2, 1536, 64, 64, 5, True, "bf16", True),
    ("f32-d64-g2-shared-noncausal", 42, 1, 4, 2, 512, 64, 128, 2, False, "f32", True),
    ("f32-d128-g2-per-head", 43, 1, 2, 1, 768, 128, 128, 4, True, "f32", False),
    # 520 blocks: the long forms of both gates (two query groups per wave
    # per head; the shared gate's two-buffer form)
    ("bf16-d128-g2-shared-520-blocks", 48, 1, 2, 1, 33280, 128, 64, 3, True, "bf16", True),
    ("bf16-d128-g2-per-head-520-blocks", 49, 1, 2, 1, 33280, 128, 64, 5, True, "bf16", False),
    ("bf16-d128-g8-shared-k17", 44, 1, 8, 1, 2048, 128, 64, 17, True, "bf16", True),
    ("bf16-d128-g2-shared-short-block", 45, 1, 4, 2, 1216, 128, 256, 3, True, "bf16", True),
    ("bf16-d128-g4-shared-topk-all", 46, 1, 4, 1, 512, 128, 64, 9, True, "bf16", True),
    ("bf16-d128-g1-shared-equals-per-head", 47, 1, 2, 2, 1024, 128, 128, 3, True, "bf16", True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gqa_parity(case):
    import sparse_long_context_moba_amd as moba
    label, seed, B, H, Hkv, S, D, Bs, top_k, causal, dtype, shared = case
    q, k, v = _inputs(seed, B, H, Hkv, S, D, Bs, dtype)
    say(f"[gpu] {label}: q={q.shape} kv={k.shape} Bs={Bs} top_k={top_k} causal={causal} shared={shared}")
    o, idx = moba.forward(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), Bs, top_k, causal,
                          gate_shared=shared)
    torch.cuda.synchronize()
    worst = _check(q, k, v, o.float().cpu().numpy(), idx.cpu().numpy(), Bs, top_k, causal, dtype, shared, label)
    say(f"[gpu] {label}: ok, max_err={worst:.3e}")


def test_gqa_equals_repeated_kv_heads():
    """A per-head gate over shared K/V gives bit-identical results to plain
    multi-head attention with each key/value head repeated for its query
    heads (same kernels, same arithmetic per query head)."""
    import sparse_long_context_moba_amd as moba
    q, k, v = _inputs(48, 1, 8, 2, 1024, 128, 128, "bf16")
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    o1, i1 = moba.forward(qd, kd, vd, 128, 3)
    kr = kd.repeat_interleave(4, dim=1).contiguous()
    vr = vd.repeat_interleave(4, dim=1).contiguous()
    o2, i2 = moba.forward(qd, kr, vr, 128, 3)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_gqa_dense_and_stages():
    """The dense kernel and the pool/select stages with key/value heads."""
    import sparse_long_context_moba_amd as moba
    q, k, v = _inputs(49, 1, 4, 2, 512, 64, 128, "f32")
    qd, kd, vd = (to_dev(x, "f32") for x in (q, k, v))
    od = moba.dense(qd, kd, vd, True).cpu().numpy()
    for h in range(4):
        ref = orc.dense_attention(q[0, h], k[0, h // 2], v[0, h // 2], True)
        assert np.abs(od[0, h] - ref).max() <= 1e-4
    kb = moba.pool(kd, 128).cpu().numpy()
    assert kb.shape == (1, 2, 4, 64)
    for hk in range(2):
        np.testing.assert_allclose(kb[0, hk], orc.pool_keys(k[0, hk], 128), rtol=1e-13, atol=1e-15)
    for shared in (False, True):
        idx = moba.select(qd, kd, 128, 2, gate_shared=shared).cpu().numpy()
        _, idx2 = moba.forward(qd, kd, vd, 128, 2, gate_shared=shared)
        np.testing.assert_array_equal(idx, idx2.cpu().numpy())


def test_gqa_varlen():
    """A varlen batch with key/value heads and a shared gate: bit-identical
    to one forward per sequence, and every row against the oracle."""
    import sparse_long_context_moba_amd as moba
    H, Hkv, D, Bs, top_k = 4, 2, 128, 128, 3
    lengths = [576, 1024, 192]
    seqs = [_inputs(50 + i, 1, H, Hkv, n, D, Bs, "bf16") for i, n in enumerate(lengths)]
    dev = [[to_dev(x, "bf16") for x in s] for s in seqs]
    qp, cu = moba.pack_varlen([d[0] for d in dev])
    kp, _ = moba.pack_varlen([d[1] for d in dev])
    vp, _ = moba.pack_varlen([d[2] for d in dev])
    o, idx = moba.forward_varlen(qp, kp, vp, cu, H, Bs, top_k, True, kv_heads=Hkv, gate_shared=True)
    torch.cuda.synchronize()
    os_ = moba.unpack_varlen(o, cu, H)
    is_ = moba.unpack_varlen(idx, cu, H)
    for i, ((q, k, v), d) in enumerate(zip(seqs, dev)):
        o1, i1 = moba.forward(d[0], d[1], d[2], Bs, top_k, True, gate_shared=True)
        assert torch.equal(is_[i], i1)
        assert torch.equal(os_[i].contiguous().view(torch.int16), o1.view(torch.int16))
        _check(q, k, v, os_[i].float().cpu().numpy(), is_[i].cpu().numpy(), Bs, top_k, True, "bf16", True,
               f"varlen seq={i}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("top_k", [3, 9])
def test_shared_gate_crowded_scores(dtype, top_k):
    """Shared gate on blocks that repeat seven patterns plus small noise:
    many rows' summed scores sit inside the fast path's rounding band and
    must be settled by the fp64 re-scoring of the summed query."""
    import sparse_long_context_moba_amd as moba
    S, D, Bs, G = 8192, 128, 64, 4
    rng = np.random.default_rng(60 + top_k)
    q = _round(rng.standard_normal((1, G, S, D)).astype(np.float32), dtype)
    pat = rng.standard_normal((7, Bs, D)).astype(np.float32)
    k = np.concatenate([pat[j % 7] for j in range(S // Bs)])[None, None]
    k = _round(k + rng.normal(0, 4e-3, k.shape).astype(np.float32), dtype)
    idx = moba.select(to_dev(q, dtype), to_dev(k, dtype), Bs, top_k, gate_shared=True).cpu().numpy()[0]
    kbar = orc.pool_keys(k[0, 0], Bs)
    qs = q[0].astype(np.float64).sum(axis=0)
    n_close = 0
    for t in range(S):
        c = t // Bs
        ref, flag, a, b = orc.select_blocks(qs[t], kbar, c, top_k, True)
        for g in range(1, G):
            assert np.array_equal(idx[g, t], idx[0, t])
        if flag:
            tau = orc.NEAR_TIE_REL * max(abs(a), abs(b))
            elig = orc.eligible_blocks(c, kbar.shape[0], True)
            s = dict(zip(elig.tolist(), (kbar[elig] @ qs[t]).tolist()))
            got = set(int(j) for j in idx[0, t] if j >= 0)
            assert c in got and len(got) == int((ref >= 0).sum())
            assert all(j in got or s[j] <= a + tau for j in s)
            assert all(j == c or s[j] >= b - tau for j in got)
        else:
            np.testing.assert_array_equal(idx[0, t], ref, err_msg=f"t={t}")
            if np.isfinite(a) and abs(a - b) < 2e-4 * max(abs(a), abs(b)):
                n_close += 1
    say(f"[gpu] shared crowded {dtype} top_k={top_k}: decided-within-2e-4={n_close}")
    assert n_close > 20
