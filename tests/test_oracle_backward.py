"""Pins for the oracle's MoBA backward (gradients with the block choice
held fixed), against facts fixed outside the oracle's backward code:
central finite differences of the oracle's own pinned forward, torch
autograd through scaled_dot_product_attention in float64 with the explicit
[S, S] mask of the chosen blocks, full-attention autograd when top_k covers
every block, and closed-form invariants of softmax attention."""
import math

import numpy as np
import pytest
import torch

from oracle import moba


def _rand(seed, S, D, Bs, bias=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, D))
    k = rng.standard_normal((S, D)) + np.repeat(rng.normal(0, bias, (-(-S // Bs), D)), Bs, axis=0)[:S]
    v = rng.standard_normal((S, D))
    do = rng.standard_normal((S, D))
    return q, k, v, do


def _mask(idx, S, Bs, causal):
    blk = np.arange(S) // Bs
    m = np.zeros((S, S), bool)
    for t in range(S):
        for j in idx[t]:
            if j >= 0:
                m[t, blk == j] = True
        if causal:
            m[t, t + 1:] = False
    return m


def _torch_grads(q, k, v, do, mask=None, causal=False):
    t = lambda x: torch.tensor(np.asarray(x, np.float64)[None, None], requires_grad=True)
    tq, tk, tv = t(q), t(k), t(v)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=None if mask is None else torch.from_numpy(mask)[None, None], is_causal=causal)
    out.backward(torch.from_numpy(np.asarray(do, np.float64))[None, None])
    return tq.grad[0, 0].numpy(), tk.grad[0, 0].numpy(), tv.grad[0, 0].numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [8, 7])
def test_backward_matches_finite_differences(causal, S):
    """dL/dx for L = sum_t o_t . do_t, o from the oracle's forward with the
    choice fixed, by central differences (a short last block when S = 7)."""
    D, Bs, top_k = 4, 2, 2
    q, k, v, do = _rand(1 + S, S, D, Bs)
    idx = moba.forward_head(q, k, v, Bs, top_k, causal)["idx"]
    dq, dk, dv, _ = moba.backward_head(q, k, v, do, idx, Bs, causal)

    def loss(q_, k_, v_):
        return sum(float(moba.attend_with_idx(q_[t], k_, v_, t, idx[t], Bs, causal) @ do[t]) for t in range(S))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for i in range(S):
            for d in range(D):
                xp, xm = x.copy(), x.copy()
                xp[i, d] += h
                xm[i, d] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                fd[i, d] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, fd, atol=1e-7, rtol=1e-6, err_msg=f"d{name}")


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_masked_autograd(causal):
    S, D, Bs, top_k = 64, 8, 8, 3
    q, k, v, do = _rand(11, S, D, Bs)
    idx = moba.forward_head(q, k, v, Bs, top_k, causal)["idx"]
    dq, dk, dv, _ = moba.backward_head(q, k, v, do, idx, Bs, causal)
    gq, gk, gv = _torch_grads(q, k, v, do, mask=_mask(idx, S, Bs, causal))
    for a, b, n in ((dq, gq, "dq"), (dk, gk, "dk"), (dv, gv, "dv")):
        np.testing.assert_allclose(a, b, atol=1e-12, err_msg=n)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_topk_covering_all_blocks_is_dense(causal):
    S, D, Bs = 48, 8, 8
    q, k, v, do = _rand(12, S, D, Bs)
    idx = moba.forward_head(q, k, v, Bs, 100, causal)["idx"]
    dq, dk, dv, _ = moba.backward_head(q, k, v, do, idx, Bs, causal)
    gq, gk, gv = _torch_grads(q, k, v, do, causal=causal)
    for a, b, n in ((dq, gq, "dq"), (dk, gk, "dk"), (dv, gv, "dv")):
        np.testing.assert_allclose(a, b, atol=1e-12, err_msg=n)


def test_backward_invariants():
    """Rows of softmax weights sum to 1 and their gradients to 0, so
    sum_u dv_u = sum_t do_t and sum_u dk_u = 0; the last key (attended only
    by the last query, causal) gets dv = p do of that query alone; constant
    values give no gradient to q or k."""
    S, D, Bs, top_k = 64, 8, 8, 2
    q, k, v, do = _rand(13, S, D, Bs)
    idx = moba.forward_head(q, k, v, Bs, top_k, True)["idx"]
    dq, dk, dv, _ = moba.backward_head(q, k, v, do, idx, Bs, True)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-11)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    keys = moba.attended_keys(S - 1, idx[S - 1], Bs, True, S)
    logits = k[keys] @ q[S - 1] / math.sqrt(D)
    p_last = np.exp(logits[-1] - logits.max()) / np.exp(logits - logits.max()).sum()
    np.testing.assert_allclose(dv[S - 1], p_last * do[S - 1], atol=1e-13)
    vc = np.tile(np.random.default_rng(14).standard_normal(D), (S, 1))
    dq0, dk0, _, _ = moba.backward_head(q, k, vc, do, idx, Bs, True)
    assert np.abs(dq0).max() < 1e-12 and np.abs(dk0).max() < 1e-12


def test_lse_matches_torch_logsumexp():
    S, D, Bs, top_k = 64, 8, 8, 3
    q, k, v, do = _rand(15, S, D, Bs)
    idx = moba.forward_head(q, k, v, Bs, top_k, True)["idx"]
    _, _, _, lse = moba.backward_head(q, k, v, do, idx, Bs, True)
    logits = torch.from_numpy(q @ k.T / math.sqrt(D))
    logits = logits.masked_fill(~torch.from_numpy(_mask(idx, S, Bs, True)), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=1).numpy(), atol=1e-12)
