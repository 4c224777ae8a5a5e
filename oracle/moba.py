"""CPU fp64 oracle for the MoBA (Mixture of Block Attention) prefill forward.

TEST INFRASTRUCTURE, not product code. Only tests/, __graft_entry__.smoke()
and bench.py's cpu_baseline leg may import or call anything in this package.
It shares no code with the HIP path (sparse_long_context_moba_amd/) and
imports nothing from it.

Sources (the web pages this method is taken from, cited by title and
section):
  [R] «MoBA 复现代码跑不通时先把本地仓库交给 Codex 读» (mhpq.cn/news/582794)
  [P] «月之暗面 MoBA 论文解读：用 TaoToken 统一 Key 跑通稀疏注意力配置骨架»
      (gsyq.cn/news/227272)
  [S] the MOBA serving article whose first heading is
      «长上下文推理为什么卡在注意力这一步» (hncyxsy.com/news/197418)

MoBA is an approximation of attention: a block-routing heuristic followed by
exact attention over the routed keys. The oracle therefore follows the
method's steps in order, in float64, one query row at a time:
  1. cut the sequence into blocks of block_size tokens ([R] §3.1, [P] §4.1);
  2. mean-pool K over each block ([P] §3.1 gating.score_fn, [S] §3; the
     serving article's §3 also names max pooling and the two combined as
     engineering options, see pool_keys);
  3. score every eligible block by the inner product of the query with the
     pooled key; blocks after the query's own block are never eligible
     ([P] §3.1 causal / mask_future, [S] §3, [R] §3.2);
  4. keep the query's own block always (its pooled mean contains future
     tokens, so it is forced rather than scored, [S] §3
     force_current_block) and fill the other top_k - 1 slots with the best
     scored blocks, ties to the lower block index ([P] §4.1 sorts block
     indices by score with a stable descending sort and keeps the first k);
  5. attend over the keys of the chosen blocks only, causal inside the
     query's own block ([S] §3), with one softmax over that whole key set.
The backward (backward_head) differentiates step 5 with the choice of
steps 3-4 held fixed (see its docstring for why that is the gradient).

Readings where the pages are silent (each is listed in the design doc):
  * top_k counts the forced current block ([P] §3.1: each query attends
    only top_k blocks; [S] §3: top-k 3 of 16 blocks is about 3/16 of the
    work);
  * gate scores are per (batch, head), raw inner products; any positive
    scale or a softmax over them is monotone and cannot change the choice;
  * top_k larger than the number of available blocks is clamped;
  * seq_len not a multiple of block_size: the block count is rounded up
    and the last block is short ([S] §4 counts blocks with a ceiling
    division; [R] §1.1's code asserts instead);
  * attention logits are scaled by 1/sqrt(head_dim);
  * non-causal mode: every other block is eligible, the own block is still
    forced, and no mask is applied inside blocks.

Parity pins for every function here live in tests/test_oracle_*.py. The
values of large workloads are not printed on the pages: their parity rests
on the oracle's definition plus those pins.
"""
from __future__ import annotations

import math

import numpy as np

NEAR_TIE_REL = 1e-5


def num_blocks(seq_len: int, block_size: int) -> int:
    """Number of key blocks ([R] §3.1: 32768 tokens in blocks of 512 -> 64).

    For a length that is not a multiple of the block size the pages
    disagree: the code in [R] §1.1 asserts, the script in [S] §4 counts
    blocks with a ceiling division. The ceiling is taken here: the last
    block holds the remaining seq_len - (n - 1) * block_size tokens.
    """
    if block_size < 1:
        raise ValueError(f"block_size must be >= 1, got {block_size}")
    if seq_len < 1:
        raise ValueError(f"seq_len must be >= 1, got {seq_len}")
    return -(-seq_len // block_size)


def block_range(j: int, seq_len: int, block_size: int) -> tuple[int, int]:
    """Token positions [lo, hi) of block j (the last block may be short)."""
    return j * block_size, min((j + 1) * block_size, seq_len)


def theoretical_sparsity(top_k: int, n_blocks: int) -> float:
    """1 - top_k / n_blocks ([P] §4.1 and §5: 64 blocks, k = 3 -> 0.953)."""
    return 1.0 - top_k / n_blocks


POOLINGS = ("mean", "max", "mean+max")


def pool_keys(k: np.ndarray, block_size: int, pooling: str = "mean") -> np.ndarray:
    """The block summary the gate scores against, per coordinate:

    - "mean": the mean of K over each block along the sequence, the paper's
      choice ([P] §3.1 mean_pool; [S] §3); a short last block is averaged
      over the tokens it holds;
    - "max": the largest value of each coordinate over the block's tokens,
      which [S] §3 names as an engineering alternative that reacts to blocks
      dense in key information;
    - "mean+max": the two combined ([S] §3 names the combination without a
      formula); read here as their sum, so a block's score is its mean
      score plus its max score.

    k: [S, D] -> [NB, D] float64.
    """
    if pooling not in POOLINGS:
        raise ValueError(f"pooling must be one of {POOLINGS}, got {pooling!r}")
    k = np.asarray(k, dtype=np.float64)
    S, D = k.shape
    nb = num_blocks(S, block_size)
    mean = np.zeros((nb, D))
    mx = np.zeros((nb, D))
    for j in range(nb):
        lo, hi = block_range(j, S, block_size)
        mean[j] = k[lo:hi].sum(axis=0) / (hi - lo)
        mx[j] = k[lo:hi].max(axis=0)
    if pooling == "mean":
        return mean
    return mx if pooling == "max" else mean + mx


def eligible_blocks(c: int, n_blocks: int, causal: bool) -> np.ndarray:
    """Blocks a query in block c may be routed to by score.

    Causal: only blocks before c ([P] §3.1, future blocks are masked).
    The own block c is never scored, only forced ([S] §3).
    """
    if causal:
        return np.arange(c, dtype=np.int64)
    return np.array([j for j in range(n_blocks) if j != c], dtype=np.int64)


def select_blocks(q_t: np.ndarray, kbar: np.ndarray, c: int, top_k: int, causal: bool):
    """Block routing for one query.

    Returns (idx, flag, a, b):
      idx  - the chosen block indices ascending, padded with -1 to top_k;
      flag - True when the last kept and the first dropped score are closer
             than NEAR_TIE_REL relative (either choice is then acceptable);
      a, b - those two scores (nan when no choice had to be made).
    """
    if top_k < 1:
        raise ValueError(f"top_k must be >= 1, got {top_k}")
    nb = kbar.shape[0]
    k_eff = min(top_k, nb)
    elig = eligible_blocks(c, nb, causal)
    scores = kbar[elig] @ np.asarray(q_t, dtype=np.float64)
    m = min(k_eff - 1, len(elig))
    # Order by score descending, then block index ascending.
    order = np.lexsort((elig, -scores))
    chosen = elig[order[:m]]
    flag, a, b = False, math.nan, math.nan
    if len(elig) > k_eff - 1 >= 1:
        a = float(scores[order[m - 1]])
        b = float(scores[order[m]])
        flag = abs(a - b) < NEAR_TIE_REL * max(abs(a), abs(b))
    sel = sorted([int(c)] + [int(j) for j in chosen])
    idx = np.full(top_k, -1, dtype=np.int64)
    idx[: len(sel)] = sel
    return idx, flag, a, b


def attended_keys(t: int, idx_row: np.ndarray, block_size: int, causal: bool,
                  seq_len: int | None = None) -> np.ndarray:
    """Key positions query t attends: every key of every chosen block (a
    short last block ends at seq_len), and inside its own block only keys
    up to t when causal ([S] §3)."""
    keys = []
    for j in idx_row:
        if j < 0:
            continue
        lo, hi = int(j) * block_size, (int(j) + 1) * block_size
        if seq_len is not None:
            hi = min(hi, seq_len)
        if causal:
            hi = min(hi, t + 1)
        keys.extend(range(lo, hi))
    return np.array(sorted(keys), dtype=np.int64)


def attend(q_t: np.ndarray, k: np.ndarray, v: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(D)) v over the given keys, float64.

    One normalisation over the whole key set; keys outside it get weight 0.
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    kk = np.asarray(k[keys], dtype=np.float64)
    vv = np.asarray(v[keys], dtype=np.float64)
    logits = kk @ q_t / math.sqrt(q_t.shape[0])
    w = np.exp(logits - logits.max())
    return (w @ vv) / w.sum()


def forward_head(q, k, v, block_size: int, top_k: int, causal: bool = True, rows=None, pooling: str = "mean"):
    """MoBA forward for one (batch, head).

    q, k, v: [S, D]. rows: query positions to evaluate (default: all).
    pooling: the block summary (see pool_keys).
    Returns dict with o [R, D] float64, idx [R, top_k] int64, flag [R] bool,
    a [R], b [R], and kbar [NB, D].
    """
    q = np.asarray(q)
    S, D = q.shape
    nb = num_blocks(S, block_size)
    if top_k < 1:
        raise ValueError(f"top_k must be >= 1, got {top_k}")
    kbar = pool_keys(k, block_size, pooling)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), D), np.float64)
    idx = np.zeros((len(rows), top_k), np.int64)
    flag = np.zeros(len(rows), bool)
    a = np.full(len(rows), np.nan)
    b = np.full(len(rows), np.nan)
    for r, t in enumerate(rows):
        c = int(t) // block_size
        idx[r], flag[r], a[r], b[r] = select_blocks(q[t], kbar, c, top_k, causal)
        o[r] = attend(q[t], k, v, attended_keys(int(t), idx[r], block_size, causal, S))
    assert nb == kbar.shape[0]
    return {"o": o, "idx": idx, "flag": flag, "a": a, "b": b, "kbar": kbar}


def forward_group(q, k, v, block_size: int, top_k: int, causal: bool = True, rows=None, pooling: str = "mean",
                  shared_gate: bool = False):
    """The query heads q [G, S, D] that read one key/value head k, v [S, D]
    (grouped-query attention; G = 1 is plain multi-head attention).

    Without a shared gate every query head routes on its own (forward_head
    with the group's K and V). With a shared gate the group routes once: a
    block's score is the sum over the group's heads of q_h . Kbar, i.e. the
    summed query against the pooled key, and every head attends the blocks
    that choice keeps ([R] §3.2 asks whether the gate is per head or shared
    across heads and leaves it open; the sum is the plainest shared score).
    Returns one forward_head-style dict per query head.
    """
    q = np.asarray(q)
    G = q.shape[0]
    if not shared_gate:
        return [forward_head(q[g], k, v, block_size, top_k, causal, rows=rows, pooling=pooling) for g in range(G)]
    S, D = q.shape[1:]
    if top_k < 1:
        raise ValueError(f"top_k must be >= 1, got {top_k}")
    kbar = pool_keys(k, block_size, pooling)
    qs = np.asarray(q, dtype=np.float64).sum(axis=0)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = [{"o": np.zeros((len(rows), D)), "idx": np.zeros((len(rows), top_k), np.int64),
            "flag": np.zeros(len(rows), bool), "a": np.full(len(rows), np.nan), "b": np.full(len(rows), np.nan),
            "kbar": kbar} for _ in range(G)]
    for r, t in enumerate(rows):
        c = int(t) // block_size
        idx, flag, a, b = select_blocks(qs[t], kbar, c, top_k, causal)
        keys = attended_keys(int(t), idx, block_size, causal, S)
        for g in range(G):
            out[g]["idx"][r], out[g]["flag"][r], out[g]["a"][r], out[g]["b"][r] = idx, flag, a, b
            out[g]["o"][r] = attend(q[g][t], k, v, keys)
    return out


def forward(q, k, v, block_size: int, top_k: int, causal: bool = True, pooling: str = "mean"):
    """Full MoBA forward over [B, H, S, D]. Returns (o float64, idx int64)."""
    B, H, S, D = q.shape
    o = np.zeros((B, H, S, D), np.float64)
    idx = np.zeros((B, H, S, top_k), np.int64)
    for bb in range(B):
        for hh in range(H):
            res = forward_head(q[bb, hh], k[bb, hh], v[bb, hh], block_size, top_k, causal, pooling=pooling)
            o[bb, hh], idx[bb, hh] = res["o"], res["idx"]
    return o, idx


def attend_with_idx(q_t, k, v, t: int, idx_row, block_size: int, causal: bool = True):
    """Attention of query t over a given block choice (forced-index mode),
    used where the GPU legitimately broke a near-tie the other way."""
    return attend(q_t, k, v, attended_keys(t, np.asarray(idx_row), block_size, causal, len(k)))


def attend_lse(q_t: np.ndarray, k: np.ndarray, keys: np.ndarray) -> float:
    """Natural-log log-sum-exp of the scaled logits q k_u / sqrt(D) over the
    attended keys: the softmax normaliser a backward pass reuses."""
    q_t = np.asarray(q_t, dtype=np.float64)
    logits = np.asarray(k[keys], dtype=np.float64) @ q_t / math.sqrt(q_t.shape[0])
    mx = logits.max()
    return float(mx + math.log(np.exp(logits - mx).sum()))


def attend_grad(q_t: np.ndarray, k: np.ndarray, v: np.ndarray, keys: np.ndarray, do_t: np.ndarray):
    """Gradients of o = softmax(l) V_U, l_u = q . k_u / sqrt(D), for an
    upstream gradient do (the textbook softmax-attention backward, float64):

        p = softmax(l);  dV_u = p_u do;  dp_u = do . v_u;
        dl_u = p_u (dp_u - do . o);  dq = sum_u dl_u k_u / sqrt(D);
        dk_u = dl_u q / sqrt(D).

    Returns (dq [D], dk [len(keys), D], dv [len(keys), D])."""
    q_t = np.asarray(q_t, dtype=np.float64)
    do_t = np.asarray(do_t, dtype=np.float64)
    kk = np.asarray(k[keys], dtype=np.float64)
    vv = np.asarray(v[keys], dtype=np.float64)
    scale = 1.0 / math.sqrt(q_t.shape[0])
    logits = kk @ q_t * scale
    w = np.exp(logits - logits.max())
    p = w / w.sum()
    o = p @ vv
    dv = np.outer(p, do_t)
    dp = vv @ do_t
    dl = p * (dp - do_t @ o)
    dq = (dl @ kk) * scale
    dk = np.outer(dl, q_t) * scale
    return dq, dk, dv


def backward_head(q, k, v, do, idx, block_size: int, causal: bool = True):
    """MoBA backward for one (batch, head): the gradients of o with respect
    to q, k and v for the upstream gradient do, with the block choice idx
    [S, top_k] (as forward_head returns it) held fixed.

    The pages use MoBA in training and fine-tuning ([S] §3 on SFT with MoBA
    layers; [P] §2) but give no gradient. Read here: the routing is a top-k
    over block scores, piecewise constant in q and k, so its derivative is
    zero wherever the choice is not tied; and the gate's scores do not
    weight the output (unchosen blocks get exactly 0, chosen ones are not
    scaled), so no gradient flows through the pooled keys. What remains is
    the gradient of one softmax attention per query over its attended keys.

    Returns (dq, dk, dv, lse): float64 [S, D] each and the per-query
    natural-log log-sum-exp [S] of the scaled logits."""
    q = np.asarray(q)
    S, D = q.shape
    dq = np.zeros((S, D))
    dk = np.zeros((S, D))
    dv = np.zeros((S, D))
    lse = np.zeros(S)
    for t in range(S):
        keys = attended_keys(t, np.asarray(idx[t]), block_size, causal, S)
        gq, gk, gv = attend_grad(q[t], k, v, keys, do[t])
        dq[t] = gq
        np.add.at(dk, keys, gk)
        np.add.at(dv, keys, gv)
        lse[t] = attend_lse(q[t], k, keys)
    return dq, dk, dv, lse


def dense_attention(q, k, v, causal: bool = True, rows=None):
    """Plain softmax attention for one head, float64, row by row."""
    S, D = q.shape
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), D), np.float64)
    for r, t in enumerate(rows):
        keys = np.arange(int(t) + 1 if causal else S, dtype=np.int64)
        out[r] = attend(q[t], k, v, keys)
    return out


def algorithmic_flops(seq_len: int, head_dim: int, block_size: int, top_k: int,
                      batch_heads: int = 1, causal: bool = True):
    """Work MoBA must do, counted from its definition.

    gate: 2*D per (query, eligible past block); attention: 4*D per
    (query, attended key). Returns (gate_flops, attn_flops, dense_flops).
    """
    S, D, Bs = seq_len, head_dim, block_size
    nb = num_blocks(S, Bs)
    if S % Bs:
        raise ValueError("the closed-form count covers whole blocks only")
    k_eff = min(top_k, nb)
    gate = 0
    keys = 0
    for c in range(nb):
        n_elig = c if causal else nb - 1
        m = min(k_eff - 1, n_elig)
        gate += Bs * n_elig
        past = m * Bs
        own = Bs * (Bs + 1) // 2 if causal else Bs * Bs
        keys += Bs * past + own
    dense_keys = S * (S + 1) // 2 if causal else S * S
    return (batch_heads * 2 * D * gate, batch_heads * 4 * D * keys,
            batch_heads * 4 * D * dense_keys)
