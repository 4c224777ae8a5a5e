"""Pins for the CPU fp64 oracle, against facts fixed outside the oracle:
numbers the pages print, hand-worked cases, brute force on tiny inputs,
library routines (torch scaled_dot_product_attention in float64) for the
cases where MoBA reduces to plain attention, and invariants of the method.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import moba


def _sdpa(q, k, v, mask=None, causal=False):
    """torch SDPA in float64 on CPU; mask: bool [S, S], True = attend."""
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask)[None, None],
        is_causal=causal)
    return out[0, 0].numpy()


def _rand_head(seed, S, D, Bs, bias=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, D))
    k = rng.standard_normal((S, D)) + np.repeat(rng.normal(0, bias, (-(-S // Bs), D)), Bs, axis=0)[:S]
    v = rng.standard_normal((S, D))
    return q, k, v


# ---------------------------------------------------------------- page numbers
def test_block_counts_printed_on_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_numbers.json")))
    for e in g["block_counts"]:
        assert moba.num_blocks(e["seq_len"], e["block_size"]) == e["n_blocks"], e["cite"]


def test_sparsity_printed_on_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_numbers.json")))
    for e in g["sparsity"]:
        s = moba.theoretical_sparsity(e["top_k"], e["n_blocks"])
        if "percent" in e:
            assert round(100 * s, e["digits"]) == e["percent"], e["cite"]
        else:
            assert round(s, e["digits"]) == e["value"], e["cite"]


def test_compute_share_printed_on_pages(golden_dir):
    """Non-causal MoBA at top_k of 16 blocks attends top_k/16 of all keys."""
    g = json.load(open(os.path.join(golden_dir, "page_numbers.json")))
    for e in g["compute_share"]:
        gate, attn, dense = moba.algorithmic_flops(e["seq_len"], 8, e["block_size"], e["top_k"],
                                                   causal=False)
        assert attn * e["share_den"] == dense * e["share_num"], e["cite"]


def test_bad_shapes_raise_naming_parameter():
    with pytest.raises(ValueError, match="block_size"):
        moba.num_blocks(100, 0)
    q, k, v = _rand_head(0, 16, 4, 4)
    with pytest.raises(ValueError, match="top_k"):
        moba.forward_head(q, k, v, 4, 0)


# -------------------------------------------------------------------- pooling
def test_pool_closed_forms():
    S, D, Bs = 48, 3, 8
    ramp = np.tile(np.arange(S, dtype=np.float64)[:, None], (1, D))
    kbar = moba.pool_keys(ramp, Bs)
    expect = np.arange(S // Bs) * Bs + (Bs - 1) / 2.0
    np.testing.assert_array_equal(kbar[:, 0], expect)
    const = np.repeat(np.arange(S // Bs, dtype=np.float64)[:, None] * 1.5 - 2, Bs, axis=0)
    const = np.tile(const, (1, D))
    np.testing.assert_array_equal(moba.pool_keys(const, Bs), np.repeat(
        (np.arange(S // Bs) * 1.5 - 2)[:, None], D, axis=1))


# ------------------------------------------------------------------- hand case
def test_hand_case(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_case.json")))
    k = np.array(g["k"], np.float64)
    v = np.array(g["v"], np.float64)
    Bs, t = g["block_size"], g["t"]
    np.testing.assert_array_equal(moba.pool_keys(k, Bs), [[2, 0], [0, 2], [1, 1], [0, 0]])
    q = np.zeros((8, 2))
    for case in g["cases"]:
        q[t] = case["q"]
        res = moba.forward_head(q, k, v, Bs, case["top_k"], True, rows=[t])
        assert list(res["idx"][0]) == case["idx"], case
        keys = moba.attended_keys(t, res["idx"][0], Bs, True)
        assert list(keys) == case["keys"]
        if "o" in case:
            np.testing.assert_allclose(res["o"][0], case["o"], atol=1e-6)
    for e in g["early_rows_top3"]:
        q[e["t"]] = e["q"]
        res = moba.forward_head(q, k, v, Bs, 3, True, rows=[e["t"]])
        assert list(res["idx"][0]) == e["idx"]
    # top_k = NB: the dense causal answer for t = 6
    q[t] = [1, 0]
    res = moba.forward_head(q, k, v, Bs, 4, True, rows=[t])
    np.testing.assert_allclose(res["o"][0], _sdpa(q, k, v, causal=True)[t], atol=1e-12)


def test_pooling_hand_case(golden_dir):
    """Mean, max and mean+max block summaries and the blocks they keep, on a
    hand-worked case where the three disagree."""
    g = json.load(open(os.path.join(golden_dir, "pooling_case.json")))
    k = np.array(g["k"], np.float64)
    Bs, t = g["block_size"], g["t"]
    v = np.zeros_like(k)
    for pooling, want in g["pooled"].items():
        np.testing.assert_array_equal(moba.pool_keys(k, Bs, pooling), want, err_msg=pooling)
    q = np.zeros((8, 2))
    for case in g["cases"]:
        q[t] = case["q"]
        for pooling, want in case["idx"].items():
            res = moba.forward_head(q, k, v, Bs, case["top_k"], True, rows=[t], pooling=pooling)
            assert list(res["idx"][0]) == want, (pooling, case)
    with pytest.raises(ValueError):
        moba.pool_keys(k, Bs, "median")


def test_max_pool_invariants():
    """The max summary against facts that hold for any block: a constant
    block gives its row, a token that dominates every coordinate is the max,
    shifting or positively scaling all keys shifts or scales the max,
    reordering tokens inside a block changes nothing, max(-k) = -min(k), and
    the max is at least the mean (strictly where a coordinate varies)."""
    rng = np.random.default_rng(3)
    Bs, nb, D = 8, 5, 6
    k = rng.standard_normal((nb * Bs, D))
    mx = moba.pool_keys(k, Bs, "max")
    const = np.repeat(rng.standard_normal((nb, D)), Bs, axis=0)
    np.testing.assert_array_equal(moba.pool_keys(const, Bs, "max"), const[::Bs])
    np.testing.assert_allclose(moba.pool_keys(const, Bs, "mean+max"), 2 * const[::Bs], rtol=1e-15, atol=1e-15)
    dom = k.copy()
    for j in range(nb):
        dom[j * Bs + (j % Bs)] = np.abs(k[j * Bs:(j + 1) * Bs]).max(axis=0) + 1.0
    np.testing.assert_array_equal(moba.pool_keys(dom, Bs, "max"), dom[[j * Bs + (j % Bs) for j in range(nb)]])
    shift = rng.standard_normal(D)
    np.testing.assert_allclose(moba.pool_keys(k + shift, Bs, "max"), mx + shift, atol=1e-12)
    np.testing.assert_allclose(moba.pool_keys(2.5 * k, Bs, "max"), 2.5 * mx, atol=1e-12)
    perm = np.concatenate([j * Bs + rng.permutation(Bs) for j in range(nb)])
    np.testing.assert_array_equal(moba.pool_keys(k[perm], Bs, "max"), mx)
    np.testing.assert_array_equal(moba.pool_keys(-k, Bs, "max"), -k.reshape(nb, Bs, D).min(axis=1))
    assert (mx > moba.pool_keys(k, Bs, "mean")).all()
    np.testing.assert_allclose(moba.pool_keys(k, Bs, "mean+max"), moba.pool_keys(k, Bs, "mean") + mx, atol=1e-12)


# ------------------------------------------------------------ short last block
def test_short_last_block_counts_and_pool():
    """A length that is not a multiple of the block size: the count rounds
    up ([S] §4's ceiling division) and the last block's summary covers only
    its own tokens. Closed forms on a ramp k_t = (t, 1)."""
    assert moba.num_blocks(100, 7) == 15
    assert moba.num_blocks(64, 8) == 8 and moba.num_blocks(65, 8) == 9 and moba.num_blocks(3, 8) == 1
    S, Bs = 20, 8
    k = np.stack([np.arange(S, dtype=np.float64), np.ones(S)], axis=1)
    np.testing.assert_array_equal(moba.pool_keys(k, Bs, "mean"), [[3.5, 1], [11.5, 1], [17.5, 1]])
    np.testing.assert_array_equal(moba.pool_keys(k, Bs, "max"), [[7, 1], [15, 1], [19, 1]])
    assert list(moba.attended_keys(19, np.array([1, 2]), Bs, False, S)) == list(range(8, 20))
    assert list(moba.attended_keys(17, np.array([0, 2]), Bs, True, S)) == list(range(0, 8)) + [16, 17]


@pytest.mark.parametrize("causal", [True, False])
def test_short_last_block_matches_masked_dense_softmax(causal):
    """The block mask built from the chosen blocks (the last block holds 4
    tokens) fed to a library attention routine."""
    S, D, Bs, top_k = 60, 8, 8, 3
    q, k, v = _rand_head(41, S, D, Bs)
    res = moba.forward_head(q, k, v, Bs, top_k, causal)
    blk = np.arange(S) // Bs
    mask = np.zeros((S, S), bool)
    for t in range(S):
        for j in res["idx"][t]:
            if j >= 0:
                mask[t, blk == j] = True
        if causal:
            mask[t, t + 1:] = False
    np.testing.assert_allclose(res["o"], _sdpa(q, k, v, mask=mask), atol=1e-12)
    full = moba.forward_head(q, k, v, Bs, 8, causal)
    np.testing.assert_allclose(full["o"], _sdpa(q, k, v, causal=causal), atol=1e-12)


def test_short_last_block_leaves_earlier_rows_alone():
    """Causal: appending a partial block changes no earlier row."""
    S, D, Bs = 60, 8, 8
    q, k, v = _rand_head(43, S, D, Bs)
    whole = moba.forward_head(q[:56], k[:56], v[:56], Bs, 3)
    ragged = moba.forward_head(q, k, v, Bs, 3)
    np.testing.assert_array_equal(ragged["idx"][:56], whole["idx"])
    np.testing.assert_allclose(ragged["o"][:56], whole["o"], atol=1e-12)
    assert (ragged["idx"][56:, :] >= -1).all() and (ragged["idx"][56:] == 7).any(axis=1).all()


# ------------------------------------------------------------------ selection
@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("causal", [True, False])
def test_selection_matches_subset_bruteforce(seed, causal):
    """Top-k by (score desc, index asc) == the max-total-score subset of size
    k-1 that is lexicographically smallest (enumerated)."""
    S, D, Bs, top_k = 56, 5, 4, 4
    q, k, v = _rand_head(seed, S, D, Bs)
    if seed % 2:  # force exact ties: duplicate a block's keys
        k[8:12] = k[20:24]
    kbar = k.reshape(-1, Bs, D).mean(axis=1)  # independent restatement of a mean
    res = moba.forward_head(q, k, v, Bs, top_k, causal)
    nb = S // Bs
    for t in range(S):
        c = t // Bs
        elig = [j for j in range(nb) if (j < c if causal else j != c)]
        m = min(top_k - 1, len(elig))
        best, best_sub = None, None
        for sub in itertools.combinations(elig, m):
            tot = sum(float(q[t] @ kbar[j]) for j in sub)
            key = (-round(tot, 9), sub)
            if best is None or key < best:
                best, best_sub = key, sub
        want = sorted(list(best_sub) + [c]) + [-1] * (top_k - 1 - m)
        assert list(res["idx"][t]) == want, (t, want)


@pytest.mark.parametrize("seed", range(4))
def test_selection_matches_pages_sort_rule(seed):
    """The pages' routing check sorts block indices by score descending with
    Python's stable sorted(..., reverse=True) and keeps the first entries
    («月之暗面 MoBA 论文解读» §4.1)."""
    S, D, Bs, top_k = 96, 8, 8, 3
    q, k, v = _rand_head(100 + seed, S, D, Bs)
    k[0:8] = k[16:24]  # exact tie between blocks 0 and 2
    res = moba.forward_head(q, k, v, Bs, top_k, True)
    kb = moba.pool_keys(k, Bs)
    for t in range(S):
        c = t // Bs
        scores = [float(q[t] @ kb[j]) for j in range(c)]
        keep = sorted(range(len(scores)), key=lambda i: scores[i], reverse=True)[: top_k - 1]
        got = [int(j) for j in res["idx"][t] if 0 <= j != c]
        assert sorted(keep) == got


def test_selection_scale_invariant():
    S, D, Bs = 64, 6, 8
    q, k, v = _rand_head(7, S, D, Bs)
    a = moba.forward_head(q, k, v, Bs, 3)["idx"]
    b = moba.forward_head(q * 3.7, k, v, Bs, 3)["idx"]
    np.testing.assert_array_equal(a, b)


def test_selection_varies_across_queries():
    """Routing is per query: with random queries the chosen sets differ
    («MoBA 复现代码跑不通…» §3.2 warns that one fixed set for every query
    points at a broadcasting bug)."""
    S, D, Bs = 256, 16, 16
    q, k, v = _rand_head(3, S, D, Bs)
    idx = moba.forward_head(q, k, v, Bs, 3)["idx"]
    late = {tuple(r) for r in idx[S - Bs:]}
    assert len(late) > 4


def test_exact_tie_prefers_lower_block_and_is_flagged():
    S, D, Bs = 32, 4, 4
    q, k, v = _rand_head(11, S, D, Bs)
    k[4:8] = k[12:16]      # blocks 1 and 3 identical
    q[28] = moba.pool_keys(k, Bs)[1] * 10  # make blocks 1 and 3 the best two
    res = moba.forward_head(q, k, v, Bs, 2, True, rows=[28])
    assert list(res["idx"][0]) == [1, 7]
    assert res["flag"][0]


# -------------------------------------------------------------------- outputs
@pytest.mark.parametrize("causal", [True, False])
def test_output_matches_masked_dense_softmax(causal):
    """Full [S, S] mask built from the chosen blocks, fed to a library
    attention routine: a different structure from the per-row oracle."""
    S, D, Bs, top_k = 64, 8, 8, 3
    q, k, v = _rand_head(5, S, D, Bs)
    res = moba.forward_head(q, k, v, Bs, top_k, causal)
    blk = np.arange(S) // Bs
    mask = np.zeros((S, S), bool)
    for t in range(S):
        for j in res["idx"][t]:
            if j >= 0:
                mask[t, blk == j] = True
        if causal:
            mask[t, t + 1:] = False
    np.testing.assert_allclose(res["o"], _sdpa(q, k, v, mask=mask), atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("top_k", [8, 9, 100])
def test_topk_at_least_blocks_is_full_attention(causal, top_k):
    S, D, Bs = 64, 8, 8
    q, k, v = _rand_head(9, S, D, Bs)
    res = moba.forward_head(q, k, v, Bs, top_k, causal)
    np.testing.assert_allclose(res["o"], _sdpa(q, k, v, causal=causal), atol=1e-12)


def test_topk1_is_block_local_causal():
    S, D, Bs = 64, 8, 16
    q, k, v = _rand_head(13, S, D, Bs)
    res = moba.forward_head(q, k, v, Bs, 1, True)
    blk = np.arange(S) // Bs
    mask = (blk[:, None] == blk[None, :]) & (np.arange(S)[None, :] <= np.arange(S)[:, None])
    np.testing.assert_allclose(res["o"], _sdpa(q, k, v, mask=mask), atol=1e-12)
    assert (res["idx"][:, 0] == blk).all()


def test_single_block_is_dense_causal():
    S, D = 40, 8
    q, k, v = _rand_head(17, S, D, S)
    res = moba.forward_head(q, k, v, S, 3, True)
    np.testing.assert_allclose(res["o"], _sdpa(q, k, v, causal=True), atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_dense_attention_matches_library_sdpa(causal):
    """The dense baseline the speedup is measured against («MoBA 复现代码跑不通…»
    §1.2: short inputs switch to plain full attention) equals torch's
    scaled_dot_product_attention in float64, causal or not, on every row and
    on a scattered subset of rows (first, last and interior ones)."""
    S, D = 72, 16
    q, k, v = _rand_head(29, S, D, 8)
    ref = _sdpa(q, k, v, causal=causal)
    np.testing.assert_allclose(moba.dense_attention(q, k, v, causal), ref, atol=1e-12)
    rows = np.array([S - 1, 0, 37, 1, 36])
    np.testing.assert_allclose(moba.dense_attention(q, k, v, causal, rows=rows), ref[rows], atol=1e-12)


def test_dense_attention_is_moba_keeping_every_block():
    """With top_k covering every block MoBA attends all keys up to the query
    (the pages' seamless switch to full attention), so it equals the dense
    baseline row for row; both are also compared with the library above."""
    S, D, Bs = 64, 8, 16
    q, k, v = _rand_head(31, S, D, Bs)
    for causal in (True, False):
        res = moba.forward_head(q, k, v, Bs, S // Bs, causal)
        np.testing.assert_allclose(moba.dense_attention(q, k, v, causal), res["o"], atol=1e-12)


def test_block_of_one_token_routes_to_best_past_tokens():
    """block_size 1: each query keeps itself plus the top_k - 1 past tokens by
    q.k (computed with torch.topk on continuous data, no ties)."""
    S, D, top_k = 48, 8, 4
    rng = np.random.default_rng(19)
    q, k, v = (rng.standard_normal((S, D)) for _ in range(3))
    res = moba.forward_head(q, k, v, 1, top_k, True)
    sc = torch.from_numpy(q @ k.T)
    mask = np.zeros((S, S), bool)
    for t in range(S):
        mask[t, t] = True
        if t:
            n = min(top_k - 1, t)
            mask[t, torch.topk(sc[t, :t], n).indices.numpy()] = True
    np.testing.assert_allclose(res["o"], _sdpa(q, k, v, mask=mask), atol=1e-12)


def test_constant_values_give_constant_output_and_convex_hull():
    S, D, Bs = 64, 8, 8
    q, k, _ = _rand_head(23, S, D, Bs)
    v = np.tile(np.linspace(-1, 2, D), (S, 1))
    res = moba.forward_head(q, k, v, Bs, 3)
    np.testing.assert_allclose(res["o"], v, atol=1e-12)
    q, k, v = _rand_head(24, S, D, Bs)
    res = moba.forward_head(q, k, v, Bs, 3)
    for t in range(S):
        keys = moba.attended_keys(t, res["idx"][t], Bs, True)
        assert (res["o"][t] <= v[keys].max(0) + 1e-12).all()
        assert (res["o"][t] >= v[keys].min(0) - 1e-12).all()


def test_no_future_leakage():
    """Changing K and V after position t leaves o_t and idx_t unchanged
    (the reason the own block is forced and masked, serving article §3)."""
    S, D, Bs = 96, 8, 8
    q, k, v = _rand_head(29, S, D, Bs)
    base = moba.forward_head(q, k, v, Bs, 3)
    rng = np.random.default_rng(1)
    for t in [0, 5, 8, 37, 63, 88]:
        k2, v2 = k.copy(), v.copy()
        k2[t + 1:] = rng.standard_normal(k2[t + 1:].shape) * 5
        v2[t + 1:] = rng.standard_normal(v2[t + 1:].shape) * 5
        r = moba.forward_head(q, k2, v2, Bs, 3, rows=[t])
        np.testing.assert_array_equal(r["idx"][0], base["idx"][t])
        np.testing.assert_allclose(r["o"][0], base["o"][t], atol=1e-12)


def test_permuting_a_past_block_changes_nothing_later():
    S, D, Bs = 96, 8, 8
    q, k, v = _rand_head(31, S, D, Bs)
    base = moba.forward_head(q, k, v, Bs, 3)
    perm = np.arange(S)
    perm[16:24] = np.random.default_rng(2).permutation(np.arange(16, 24))
    r = moba.forward_head(q, k[perm], v[perm], Bs, 3)
    np.testing.assert_array_equal(r["idx"][24:], base["idx"][24:])
    np.testing.assert_allclose(r["o"][24:], base["o"][24:], atol=1e-12)


def test_algorithmic_flops_against_counted_keys():
    S, D, Bs, top_k = 64, 8, 8, 3
    q, k, v = _rand_head(37, S, D, Bs)
    res = moba.forward_head(q, k, v, Bs, top_k)
    keys = sum(len(moba.attended_keys(t, res["idx"][t], Bs, True)) for t in range(S))
    gate_pairs = sum(t // Bs for t in range(S))
    g, a, d = moba.algorithmic_flops(S, D, Bs, top_k)
    assert a == 4 * D * keys and g == 2 * D * gate_pairs and d == 4 * D * S * (S + 1) // 2


# --------------------------------------------------------------- input recipe
def test_synth_is_deterministic_and_bf16_rounding_matches_torch():
    w = synth.WORKLOADS["headline_32k"]
    a = synth.make_head(w.seed, 0, 3, 1024, 128, 512, "bf16")
    b = synth.make_head(w.seed, 0, 3, 1024, 128, 512, "bf16")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    raw = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    mine = synth.round_to_bf16(raw)
    ref = torch.from_numpy(raw).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(mine, ref)
    bits = synth.bf16_bits(mine)
    back = torch.from_numpy(bits).view(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(back, mine)


def test_sample_rows_contains_edges():
    w = synth.WORKLOADS["headline_32k"]
    rows = synth.sample_rows(w, 4096)
    assert len(rows) == 4096 and len({tuple(r) for r in rows}) == 4096
    s = {tuple(r) for r in rows}
    for t in [0, 511, 512, 32767, 32768 - 512]:
        assert (0, 0, t) in s and (0, 31, t) in s


# --------------------------------------------------- grouped heads, shared gate
def test_group_without_shared_gate_is_per_head():
    S, D, Bs = 64, 8, 8
    rng = np.random.default_rng(51)
    q = rng.standard_normal((3, S, D))
    _, k, v = _rand_head(51, S, D, Bs)
    out = moba.forward_group(q, k, v, Bs, 3, True)
    for g in range(3):
        ref = moba.forward_head(q[g], k, v, Bs, 3, True)
        np.testing.assert_array_equal(out[g]["idx"], ref["idx"])
        np.testing.assert_array_equal(out[g]["o"], ref["o"])


@pytest.mark.parametrize("causal", [True, False])
def test_shared_gate_matches_subset_bruteforce(causal):
    """The shared choice maximises the group's total score: enumerate every
    (k-1)-subset of eligible blocks and sum q_h . Kbar_j over heads and
    blocks term by term."""
    S, D, Bs, top_k, G = 48, 4, 8, 3, 3
    rng = np.random.default_rng(53)
    q = rng.standard_normal((G, S, D))
    _, k, v = _rand_head(53, S, D, Bs)
    out = moba.forward_group(q, k, v, Bs, top_k, causal, shared_gate=True)
    kbar = k.reshape(S // Bs, Bs, D).mean(axis=1)
    for t in range(S):
        c = t // Bs
        elig = [j for j in range(S // Bs) if (j < c if causal else j != c)]
        m = min(top_k - 1, len(elig))
        best, best_set = None, None
        for sub in itertools.combinations(elig, m):
            tot = sum(float(q[g, t] @ kbar[j]) for g in range(G) for j in sub)
            if best is None or tot > best + 1e-12:
                best, best_set = tot, sub
        want = sorted(set(best_set) | {c})
        for g in range(G):
            assert [int(x) for x in out[g]["idx"][t] if x >= 0] == want, (t, g)


def test_shared_gate_special_cases():
    """One head: the shared gate is the head's own. Identical heads: the
    summed query is a positive multiple of each, so the choice is each
    head's own. Every head attends with its own query."""
    S, D, Bs = 64, 8, 8
    rng = np.random.default_rng(55)
    q1 = rng.standard_normal((1, S, D))
    _, k, v = _rand_head(55, S, D, Bs)
    one = moba.forward_group(q1, k, v, Bs, 3, True, shared_gate=True)[0]
    ref = moba.forward_head(q1[0], k, v, Bs, 3, True)
    np.testing.assert_array_equal(one["idx"], ref["idx"])
    np.testing.assert_allclose(one["o"], ref["o"], atol=1e-12)
    same = np.repeat(q1, 4, axis=0)
    out = moba.forward_group(same, k, v, Bs, 3, True, shared_gate=True)
    for g in range(4):
        np.testing.assert_array_equal(out[g]["idx"], ref["idx"])
    # top_k >= n_blocks: every head gets full causal attention with its own query
    q3 = rng.standard_normal((3, S, D))
    full = moba.forward_group(q3, k, v, Bs, 8, True, shared_gate=True)
    for g in range(3):
        np.testing.assert_allclose(full[g]["o"], _sdpa(q3[g], k, v, causal=True), atol=1e-12)
