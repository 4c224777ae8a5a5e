"""The oracle's pins catch plausible mistakes.

Each case plants one bug in the oracle on the CPU (one function of
oracle.moba is swapped for a wrong copy for the duration of the case) and
runs the pin tests of test_oracle_pins.py against it; at least one of them
must fail. The oracle itself is never modified on disk, and every swap is
undone before the next case. A case that no pin detects means a pin is
missing."""
import contextlib
import math
import os

import numpy as np
import pytest

from oracle import moba
from tests import test_oracle_backward as bwd
from tests import test_oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _pins():
    """(name, callable) for every pin that exercises the method's steps."""
    yield "hand_case", lambda: pins.test_hand_case(GOLDEN)
    yield "pool_closed_forms", pins.test_pool_closed_forms
    yield "pooling_hand_case", lambda: pins.test_pooling_hand_case(GOLDEN)
    yield "max_pool_invariants", pins.test_max_pool_invariants
    yield "short_block_pool", pins.test_short_last_block_counts_and_pool
    for causal in (True, False):
        yield f"short_block_dense[{causal}]", lambda c=causal: pins.test_short_last_block_matches_masked_dense_softmax(c)
    yield "short_block_earlier_rows", pins.test_short_last_block_leaves_earlier_rows_alone
    yield "group_per_head", pins.test_group_without_shared_gate_is_per_head
    for causal in (True, False):
        yield f"shared_gate_bruteforce[{causal}]", lambda c=causal: pins.test_shared_gate_matches_subset_bruteforce(c)
    yield "shared_gate_special", pins.test_shared_gate_special_cases
    yield "backward_finite_differences", lambda: bwd.test_backward_matches_finite_differences(True, 8)
    for causal in (True, False):
        yield f"backward_masked_autograd[{causal}]", lambda c=causal: bwd.test_backward_matches_masked_autograd(c)
    yield "backward_dense", lambda: bwd.test_backward_topk_covering_all_blocks_is_dense(True)
    yield "backward_invariants", bwd.test_backward_invariants
    yield "backward_lse", bwd.test_lse_matches_torch_logsumexp
    for seed in range(6):
        for causal in (True, False):
            yield f"subset_bruteforce[{seed},{causal}]", (
                lambda s=seed, c=causal: pins.test_selection_matches_subset_bruteforce(s, c))
    for seed in range(4):
        yield f"pages_sort_rule[{seed}]", lambda s=seed: pins.test_selection_matches_pages_sort_rule(s)
    yield "exact_tie", pins.test_exact_tie_prefers_lower_block_and_is_flagged
    for causal in (True, False):
        yield f"masked_dense[{causal}]", lambda c=causal: pins.test_output_matches_masked_dense_softmax(c)
        for top_k in (8, 9, 100):
            yield f"topk_ge_nb[{causal},{top_k}]", (
                lambda c=causal, k=top_k: pins.test_topk_at_least_blocks_is_full_attention(c, k))
    yield "topk1_local", pins.test_topk1_is_block_local_causal
    for causal in (True, False):
        yield f"dense_sdpa[{causal}]", lambda c=causal: pins.test_dense_attention_matches_library_sdpa(c)
    yield "dense_is_moba_all_blocks", pins.test_dense_attention_is_moba_keeping_every_block
    yield "single_block_dense", pins.test_single_block_is_dense_causal
    yield "block_of_one_token", pins.test_block_of_one_token_routes_to_best_past_tokens
    yield "constant_values", pins.test_constant_values_give_constant_output_and_convex_hull
    yield "no_future_leakage", pins.test_no_future_leakage
    yield "permute_past_block", pins.test_permuting_a_past_block_changes_nothing_later


@contextlib.contextmanager
def planted(name, fn):
    old = getattr(moba, name)
    setattr(moba, name, fn)
    try:
        yield
    finally:
        setattr(moba, name, old)


def _failing_pins():
    failed = []
    for name, pin in _pins():
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


# ---------------------------------------------------------------- the bugs
_orig_pool = moba.pool_keys
_orig_elig = moba.eligible_blocks
_orig_select = moba.select_blocks
_orig_keys = moba.attended_keys
_orig_attend = moba.attend
_orig_grad = moba.attend_grad
_orig_lse = moba.attend_lse
_orig_dense = moba.dense_attention


def pool_wrong_denominator(k, block_size, pooling="mean"):
    # mean over Bs - 1 (an off-by-one denominator)
    return _orig_pool(k, block_size, pooling) * block_size / max(block_size - 1, 1)


def pool_first_key_only(k, block_size, pooling="mean"):
    k = np.asarray(k, dtype=np.float64)
    return k[::block_size].copy()


def num_blocks_floor(seq_len, block_size):
    # a short last block silently dropped
    if block_size < 1:
        raise ValueError("block_size")
    return seq_len // block_size


def pool_short_block_over_block_size(k, block_size, pooling="mean"):
    # the short last block's mean divided by block_size instead of its length
    out = _orig_pool(k, block_size, pooling)
    S = np.asarray(k).shape[0]
    L = S - (out.shape[0] - 1) * block_size
    if pooling == "mean" and L < block_size:
        out[-1] *= L / block_size
    return out


_orig_group = moba.forward_group


def shared_gate_first_head(q, k, v, block_size, top_k, causal=True, rows=None, pooling="mean", shared_gate=False):
    # the shared choice taken from the first head's query alone
    if not shared_gate:
        return _orig_group(q, k, v, block_size, top_k, causal, rows, pooling, False)
    q = np.asarray(q)
    lead = _orig_group(q[:1], k, v, block_size, top_k, causal, rows, pooling, True)[0]
    out = []
    for g in range(q.shape[0]):
        r = dict(lead)
        keys_rows = rows if rows is not None else np.arange(q.shape[1])
        r["o"] = np.array([moba.attend(q[g][t], k, v, moba.attended_keys(int(t), lead["idx"][i], block_size, causal,
                                                                            q.shape[1]))
                           for i, t in enumerate(keys_rows)])
        out.append(r)
    return out


def shared_gate_ignored(q, k, v, block_size, top_k, causal=True, rows=None, pooling="mean", shared_gate=False):
    # every head routes on its own even when the gate is shared
    return _orig_group(q, k, v, block_size, top_k, causal, rows, pooling, False)


def pool_max_is_min(k, block_size, pooling="mean"):
    # a sign slip in the max reduction
    if pooling == "mean":
        return _orig_pool(k, block_size)
    k = np.asarray(k, dtype=np.float64)
    mn = k.reshape(-1, block_size, k.shape[1]).min(axis=1)
    return mn if pooling == "max" else _orig_pool(k, block_size) + mn


def pool_max_over_dims(k, block_size, pooling="mean"):
    # the max taken across coordinates instead of across the block's tokens
    if pooling == "mean":
        return _orig_pool(k, block_size)
    k = np.asarray(k, dtype=np.float64)
    blocks = k.reshape(-1, block_size, k.shape[1])
    mx = np.repeat(blocks.max(axis=2).max(axis=1, keepdims=True), k.shape[1], axis=1)
    return mx if pooling == "max" else _orig_pool(k, block_size) + mx


def pool_combined_is_max(k, block_size, pooling="mean"):
    # mean+max read as the max alone
    return _orig_pool(k, block_size, "max" if pooling == "mean+max" else pooling)


def eligible_includes_own(c, n_blocks, causal):
    # the own block is scored as well as forced
    if causal:
        return np.arange(c + 1, dtype=np.int64)
    return np.arange(n_blocks, dtype=np.int64)


def eligible_includes_next(c, n_blocks, causal):
    # the block after the own block leaks in (future routing)
    e = list(_orig_elig(c, n_blocks, causal))
    if causal and c + 1 < n_blocks:
        e.append(c + 1)
    return np.array(e, dtype=np.int64)


def select_ties_to_higher_index(q_t, kbar, c, top_k, causal):
    nb = kbar.shape[0]
    k_eff = min(top_k, nb)
    elig = moba.eligible_blocks(c, nb, causal)
    scores = kbar[elig] @ np.asarray(q_t, dtype=np.float64)
    m = min(k_eff - 1, len(elig))
    order = np.lexsort((-elig, -scores))  # higher index first among equal scores
    chosen = elig[order[:m]]
    flag, a, b = False, math.nan, math.nan
    if len(elig) > k_eff - 1 >= 1:
        a, b = float(scores[order[m - 1]]), float(scores[order[m]])
        flag = abs(a - b) < moba.NEAR_TIE_REL * max(abs(a), abs(b))
    sel = sorted([int(c)] + [int(j) for j in chosen])
    idx = np.full(top_k, -1, dtype=np.int64)
    idx[: len(sel)] = sel
    return idx, flag, a, b


def select_topk_excludes_own(q_t, kbar, c, top_k, causal):
    # top_k read as "k past blocks plus the own block"
    idx, flag, a, b = _orig_select(q_t, kbar, c, top_k + 1, causal)
    return idx[:top_k], flag, a, b


def select_lowest_scores(q_t, kbar, c, top_k, causal):
    # a sign slip: the worst blocks are kept
    return _orig_select(-np.asarray(q_t, dtype=np.float64), kbar, c, top_k, causal)


def keys_no_causal_mask(t, idx_row, block_size, causal, seq_len=None):
    return _orig_keys(t, idx_row, block_size, False, seq_len)


def keys_drop_own_block(t, idx_row, block_size, causal, seq_len=None):
    # the own block's keys are left out (kept only when nothing else is chosen)
    c = t // block_size
    past = [int(j) for j in idx_row if j >= 0 and j != c]
    return _orig_keys(t, np.array(past if past else list(idx_row)), block_size, causal, seq_len)


def attend_no_scale(q_t, k, v, keys):
    q_t = np.asarray(q_t, dtype=np.float64)
    return _orig_attend(q_t * math.sqrt(q_t.shape[0]), k, v, keys)


def attend_scale_by_d(q_t, k, v, keys):
    q_t = np.asarray(q_t, dtype=np.float64)
    return _orig_attend(q_t / math.sqrt(q_t.shape[0]), k, v, keys)


def attend_unnormalised(q_t, k, v, keys):
    q_t = np.asarray(q_t, dtype=np.float64)
    kk, vv = np.asarray(k[keys], np.float64), np.asarray(v[keys], np.float64)
    logits = kk @ q_t / math.sqrt(q_t.shape[0])
    return np.exp(logits - logits.max()) @ vv


def dense_drops_diagonal(q, k, v, causal=True, rows=None):
    # each query attends only the keys before it, not itself
    S, D = q.shape
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), D))
    for r, t in enumerate(rows):
        out[r] = moba.attend(q[t], k, v, np.arange(int(t) if causal else S, dtype=np.int64))
    return out


def dense_ignores_causal(q, k, v, causal=True, rows=None):
    return _orig_dense(q, k, v, False, rows)


def dense_ignores_rows(q, k, v, causal=True, rows=None):
    # the requested rows are evaluated as if they were the first ones
    n = q.shape[0] if rows is None else len(rows)
    return _orig_dense(q, k, v, causal)[:n]


def _grad_parts(q_t, k, v, keys, do_t):
    q_t = np.asarray(q_t, dtype=np.float64)
    do_t = np.asarray(do_t, dtype=np.float64)
    kk, vv = np.asarray(k[keys], np.float64), np.asarray(v[keys], np.float64)
    scale = 1.0 / math.sqrt(q_t.shape[0])
    logits = kk @ q_t * scale
    w = np.exp(logits - logits.max())
    return q_t, do_t, kk, vv, scale, w, w / w.sum()


def grad_drop_delta(q_t, k, v, keys, do_t):
    # the softmax Jacobian's do . o term is dropped
    q_t, do_t, kk, vv, scale, w, p = _grad_parts(q_t, k, v, keys, do_t)
    dl = p * (vv @ do_t)
    return (dl @ kk) * scale, np.outer(dl, q_t) * scale, np.outer(p, do_t)


def grad_dq_unscaled(q_t, k, v, keys, do_t):
    dq, dk, dv = _orig_grad(q_t, k, v, keys, do_t)
    return dq * math.sqrt(np.asarray(q_t).shape[0]), dk, dv


def grad_dv_unnormalised(q_t, k, v, keys, do_t):
    q_t, do_t, kk, vv, scale, w, p = _grad_parts(q_t, k, v, keys, do_t)
    dq, dk, _ = _orig_grad(q_t, k, v, keys, do_t)
    return dq, dk, np.outer(w, do_t)


def grad_dk_from_keys(q_t, k, v, keys, do_t):
    # dk built from the keys instead of the query
    q_t, do_t, kk, vv, scale, w, p = _grad_parts(q_t, k, v, keys, do_t)
    dq, _, dv = _orig_grad(q_t, k, v, keys, do_t)
    dl = p * (vv @ do_t - do_t @ (p @ vv))
    return dq, dl[:, None] * kk * scale, dv


def lse_unscaled(q_t, k, keys):
    q_t = np.asarray(q_t, dtype=np.float64)
    return _orig_lse(q_t * math.sqrt(q_t.shape[0]), k, keys)


MUTATIONS = [
    ("dense_attention", dense_drops_diagonal),
    ("dense_attention", dense_ignores_causal),
    ("dense_attention", dense_ignores_rows),
    ("attend_grad", grad_drop_delta),
    ("attend_grad", grad_dq_unscaled),
    ("attend_grad", grad_dv_unnormalised),
    ("attend_grad", grad_dk_from_keys),
    ("attend_lse", lse_unscaled),
    ("pool_keys", pool_wrong_denominator),
    ("pool_keys", pool_first_key_only),
    ("pool_keys", pool_max_is_min),
    ("num_blocks", num_blocks_floor),
    ("forward_group", shared_gate_first_head),
    ("forward_group", shared_gate_ignored),
    ("pool_keys", pool_short_block_over_block_size),
    ("pool_keys", pool_max_over_dims),
    ("pool_keys", pool_combined_is_max),
    ("eligible_blocks", eligible_includes_own),
    ("eligible_blocks", eligible_includes_next),
    ("select_blocks", select_ties_to_higher_index),
    ("select_blocks", select_topk_excludes_own),
    ("select_blocks", select_lowest_scores),
    ("attended_keys", keys_no_causal_mask),
    ("attended_keys", keys_drop_own_block),
    ("attend", attend_no_scale),
    ("attend", attend_scale_by_d),
    ("attend", attend_unnormalised),
]


def test_unmodified_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f.__name__ for _, f in MUTATIONS])
def test_planted_mistake_is_caught(name, fn):
    with planted(name, fn):
        failed = _failing_pins()
    assert failed, f"no pin detects {fn.__name__} in {name}"
