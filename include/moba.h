/*
 * moba.h — C ABI of libmoba.so, the MI355X (gfx950) MoBA prefill forward.
 *
 * MoBA (Mixture of Block Attention) cuts K into blocks of block_size
 * tokens, pools each block (by default its mean; see moba_pooling_t), lets
 * every query score the eligible blocks
 * by the inner product with the pooled key, always keeps the query's own
 * block, keeps the top_k blocks in total, and runs softmax attention over
 * the keys of the chosen blocks only (causal inside the own block).
 * Sources, cited by page title and section:
 *   [R] «MoBA 复现代码跑不通时先把本地仓库交给 Codex 读» (mhpq.cn)
 *   [P] «月之暗面 MoBA 论文解读：用 TaoToken 统一 Key 跑通稀疏注意力配置骨架» (gsyq.cn)
 *   [S] MOBA serving article, first heading «长上下文推理为什么卡在注意力这一步» (hncyxsy.com)
 *
 * Conventions for every entry point:
 *   - Tensors q and o are [batch, heads, seq_len, head_dim]; k and v are
 *     [batch, kv_heads, seq_len, head_dim] (kv_heads = heads unless the
 *     problem says otherwise, see moba_problem_t). All are contiguous,
 *     row-major, in device memory, of the problem's dtype (fp32 or bf16).
 *   - block_idx is int32 [batch, heads, seq_len, top_k] in device memory.
 *   - The caller owns every buffer, including the workspace; the library
 *     never allocates device memory and keeps no per-call state (one
 *     exception: moba_forward_noalloc works in a scratch array compiled
 *     into the library, see there).
 *   - stream is a hipStream_t (NULL = the null stream). Work is queued on
 *     it and the call returns without synchronising; a device fault shows
 *     at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched. On
 *     error nothing is launched and no output is touched; the returned code
 *     names the class of error and moba_last_error() (per calling thread)
 *     names the parameter.
 *   - Results are deterministic: the same inputs give bit-identical o and
 *     block_idx on every call.
 *   - Calls on different streams with distinct workspaces may run
 *     concurrently.
 */
#ifndef MOBA_H
#define MOBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOBA_ABI_VERSION 7

typedef enum { MOBA_F32 = 0, MOBA_BF16 = 1 } moba_dtype_t;

/* The block summary the gate scores each block against ([P] §3.1 uses the
 * mean of the block's keys along the sequence; [S] §3 names max pooling and
 * the two combined as engineering options). Per coordinate:
 *   MOBA_POOL_MEAN     — mean over the block's tokens (the paper's gate);
 *   MOBA_POOL_MAX      — largest value over the block's tokens;
 *   MOBA_POOL_MEAN_MAX — mean + max (the combination, read as their sum). */
typedef enum { MOBA_POOL_MEAN = 0, MOBA_POOL_MAX = 1, MOBA_POOL_MEAN_MAX = 2 } moba_pooling_t;

typedef enum {
  MOBA_OK = 0,
  MOBA_ERR_NULL = 1,        /* a required pointer is NULL */
  MOBA_ERR_SHAPE = 2,       /* non-positive size; heads not a multiple of kv_heads */
  MOBA_ERR_ARG = 3,         /* top_k < 1, pooling unknown, a reserved field != 0 */
  MOBA_ERR_DTYPE = 4,       /* dtype is neither MOBA_F32 nor MOBA_BF16 */
  MOBA_ERR_UNSUPPORTED = 5, /* valid MoBA problem outside this build's kernel limits */
  MOBA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than moba_workspace_size */
  MOBA_ERR_DEVICE = 7       /* a HIP call or kernel launch failed */
} moba_status_t;

/* One MoBA problem.
 *   block_size — tokens per key block ([R] §3.1, [P] §3.1). n_blocks =
 *                ceil(seq_len / block_size): when seq_len is not a multiple
 *                of it the last block holds the remaining tokens and its
 *                summary covers only them ([S] §4 counts blocks with a
 *                ceiling division; [R] §1.1's code asserts instead).
 *   top_k      — blocks each query attends, counting its own forced block
 *                ([P] §3.1, [S] §3). top_k > n_blocks is clamped,
 *                so top_k >= the block count gives full attention.
 *   causal     — nonzero: only blocks before the query's own block may be
 *                chosen and the own block is causally masked ([P] §3.1
 *                causal / mask_future, [S] §3). Zero: every other block is
 *                eligible and no mask is applied inside blocks.
 *   dtype      — moba_dtype_t of q, k, v and o. Arithmetic accumulates in
 *                fp32; o is rounded to the dtype (nearest, ties to even).
 *   kv_heads   — key/value heads (grouped-query attention): query head h
 *                reads key/value head h / (heads / kv_heads), so heads must
 *                be a multiple of it. 0 means kv_heads = heads (plain
 *                multi-head attention). The block summaries are pooled
 *                once per key/value head.
 *   gate_shared— zero: every query head routes on its own scores. Nonzero:
 *                the query heads of one key/value head route together on
 *                the sum of their scores, sum_h q_h . kbar_j (the same as
 *                the summed query against the pooled key), and all of them
 *                attend the blocks that choice keeps, each with its own
 *                query. ([R] §3.2 asks whether the gate is per head or
 *                shared across heads and leaves it open; the sum is the
 *                plain shared score.) block_idx then repeats the group's
 *                choice in each of its query heads' rows.
 * Any seq_len >= 1 is accepted: the last block, and the last tile of
 * queries and keys, may be partial (padding rows are masked, and loads
 * never leave the sequence).
 * Kernel limits of this build (MOBA_ERR_UNSUPPORTED otherwise):
 *   head_dim in {64, 128}; block_size a multiple of 64;
 *   min(top_k, n_blocks) - 1 <= 16 unless top_k >= n_blocks;
 *   seq_len < 2^27; heads * blocks over the batch < 2^31;
 *   heads * tokens over the batch * (min(top_k, n_blocks) - 1) < 2^31. */
typedef struct {
  int64_t batch;
  int64_t heads;
  int64_t seq_len;
  int64_t head_dim;
  int64_t block_size;
  int64_t top_k;
  int32_t causal;
  int32_t dtype;
  int32_t pooling;  /* moba_pooling_t; a zeroed field selects the mean */
  int32_t reserved; /* must be 0 */
  int64_t kv_heads; /* 0 = heads; otherwise a divisor of heads */
  int32_t gate_shared; /* 0 = per-head gate */
  int32_t reserved2;   /* must be 0 */
} moba_problem_t;

/* MOBA_ABI_VERSION of the loaded library. */
int moba_abi_version(void);

/* Static text for a status code (never NULL). */
const char* moba_status_str(moba_status_t status);

/* Detail of the last failing call on this thread, naming the bad
 * parameter ("" after a successful call). Valid until the next call. */
const char* moba_last_error(void);

/* Bytes of device workspace moba_forward needs for *p (host only, no HIP
 * call). Fails with the same codes as moba_forward's validation. */
moba_status_t moba_workspace_size(const moba_problem_t* p, size_t* bytes);

/* MoBA prefill forward ([P] §3.1, [S] §3; steps listed at the top).
 *   q, k, v  — inputs (see conventions); read only.
 *   o        — output attention, same shape and dtype as q.
 *   block_idx— output, per query the chosen block indices in ascending order
 *              (own block included), padded with -1 up to top_k entries.
 *              Among equal gate scores the lower block index is kept (the
 *              pages' routing check sorts with a stable descending sort,
 *              [P] §4.1).
 *   workspace— device scratch of at least moba_workspace_size bytes,
 *              256-byte aligned; its contents on entry do not matter and
 *              are left undefined.
 * Gate scores are selected exactly: a query whose fast (MFMA) scores leave
 * the cut between kept and dropped blocks inside their rounding bound is
 * re-scored in fp64. */
moba_status_t moba_forward(const moba_problem_t* p, const void* q, const void* k, const void* v,
                 void* o, int32_t* block_idx, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Bytes of the device scratch array moba_forward_noalloc works in (one
 * copy per GPU the library runs on, held until the process ends). */
#define MOBA_NOALLOC_SCRATCH_BYTES (256u << 20)

/* moba_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the workspace taken from a scratch
 * array compiled into the library instead of a caller buffer. The call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the array's device address on the calling thread's current
 * device (which must be the stream's device) is looked up on that device's
 * first call and kept.
 *   q, k, v, o, block_idx, stream — as for moba_forward.
 * Limit: problems whose moba_workspace_size exceeds
 * MOBA_NOALLOC_SCRATCH_BYTES fail with MOBA_ERR_WORKSPACE before anything
 * is launched (256 MiB holds, for example, 32 heads x 8192 tokens or
 * 8 heads x 32768 tokens at head_dim 128, block 512, top_k 3, bf16).
 * Every call on one GPU shares that GPU's array and nothing in it has to
 * start cleared (the forward writes each byte it reads); calls that overlap
 * on one GPU (different streams or threads without ordering between them)
 * race on it and must be serialised by the caller. */
moba_status_t moba_forward_noalloc(const moba_problem_t* p, const void* q, const void* k, const void* v,
                                   void* o, int32_t* block_idx, void* stream);

/* moba_forward that also writes, per query, the natural-log log-sum-exp of
 * its scaled logits q.k_u / sqrt(head_dim) over every key it attended (the
 * softmax normaliser a backward pass reuses).
 *   lse — device float32 [batch, heads, seq_len]; must not be NULL.
 * Everything else as moba_forward (same workspace size). */
moba_status_t moba_forward_lse(const moba_problem_t* p, const void* q, const void* k, const void* v,
                     void* o, int32_t* block_idx, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream);

/* MoBA backward (bf16 inputs only; MOBA_ERR_UNSUPPORTED otherwise; any
 * seq_len, as the forward): the
 * gradients of o with respect to q, k and v for the upstream gradient dout,
 * with the forward's block choice held fixed. The routing is a top-k over
 * block scores, constant between ties, and the gate's scores do not weight
 * the output, so no gradient flows through the block summaries; what
 * remains is, per query, the gradient of one softmax attention over its
 * attended keys. MoBA is used in training and fine-tuning ([S] §3, [P] §2);
 * the pages give no gradient, this is the plain reading.
 *   q, k, v, o, block_idx — the forward's inputs and outputs (same problem).
 *           A block_idx row is read up to its first -1; entries that do not
 *           name a past block the query may attend (outside 0..n_blocks-1,
 *           its own block, a later block under causal routing) are
 *           skipped, and only the first min(top_k, n_blocks) - 1 (at most
 *           the eligible count) past entries are used. The own block is
 *           always attended. A row the forward wrote is used as is; an
 *           edited row gets the gradient of the blocks that remain, which
 *           is that of the forward only if lse matches them;
 *   lse   — device float32 [batch, heads, seq_len] from moba_forward_lse;
 *   dout  — device, like o: the upstream gradient;
 *   dq    — output, like q; dk, dv — outputs, like k and v (summed over the
 *           query heads of each key/value head).
 *   workspace — at least moba_backward_workspace_size bytes, 256-byte
 *           aligned, contents on entry irrelevant.
 * Deterministic: no floating-point atomics; dq sums its per-block parts in
 * a fixed order. */
moba_status_t moba_backward_workspace_size(const moba_problem_t* p, size_t* bytes);
moba_status_t moba_backward(const moba_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const int32_t* block_idx, const float* lse, void* dq, void* dk,
                  void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Varlen batch: n_seqs independent sequences of different lengths in one
 * call, each routed and attended on its own, blocks starting at its first
 * token (the per-sequence cu_seqlens packing the pages describe for
 * flash-attn, [R] §3.3). The batch runs as one launch chain, the same
 * kernels and launch count as a single sequence: every kernel finds its
 * sequence in a small table of per-sequence prefix sums (tokens, blocks,
 * tiles) that the call copies into the workspace.
 *   cu_seqlens — HOST int64 [n_seqs + 1]: cu_seqlens[0] = 0 and sequence i
 *                holds tokens cu_seqlens[i] .. cu_seqlens[i+1] - 1; every
 *                length must be >= 1 (any length; a short last block and
 *                a partial last tile are allowed) and below 2^27.
 *   p          — heads, kv_heads, head_dim, block_size, top_k, causal,
 *                dtype, pooling and gate_shared for every sequence; p->batch must equal n_seqs and
 *                p->seq_len the total cu_seqlens[n_seqs] (both checked).
 *   q, o       — the sequences back to back, sequence i stored as
 *                [heads, len_i, head_dim] contiguous from element
 *                cu_seqlens[i] * heads * head_dim.
 *   k, v       — likewise with kv_heads: sequence i as [kv_heads, len_i,
 *                head_dim] from element cu_seqlens[i] * kv_heads * head_dim.
 *   block_idx  — likewise, sequence i as [heads, len_i, top_k] from element
 *                cu_seqlens[i] * heads * top_k.
 *   workspace  — at least moba_workspace_size_varlen bytes (the lists and
 *                partials of all sequences at once, plus the table).
 * Every sequence is validated before anything is launched; an error names
 * the sequence. The table goes to the device with hipMemcpyAsync from host
 * memory (ordered on the stream). */
moba_status_t moba_workspace_size_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs,
                               size_t* bytes);
moba_status_t moba_forward_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs,
                        const void* q, const void* k, const void* v, void* o, int32_t* block_idx,
                        void* workspace, size_t workspace_bytes, void* stream);

/* moba_forward_varlen plus each query's natural-log log-sum-exp (as
 * moba_forward_lse), for moba_backward_varlen.
 *   lse — device float32, sequence i as [heads, len_i] from element
 *         cu_seqlens[i] * heads; must not be NULL.
 * Everything else as moba_forward_varlen (same workspace size). */
moba_status_t moba_forward_varlen_lse(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs,
                            const void* q, const void* k, const void* v, void* o, int32_t* block_idx,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* MoBA backward of a varlen batch: each sequence's dq, dk, dv exactly as
 * moba_backward computes them for that sequence alone (sequences never
 * interact: the cu_seqlens packing of [R] §3.3). Sequence i is the uniform
 * problem of batch 1 and seq_len len_i at its offset; the sequences run one
 * after another on the stream, each a launch chain of its own, reusing the
 * workspace.
 *   cu_seqlens, p — as moba_forward_varlen; bf16 inputs (an error names
 *           the first sequence the backward rejects);
 *   q, k, v, o, dout, dq — the sequences back to back as q in
 *           moba_forward_varlen; dk, dv as k and v there;
 *   block_idx, lse — from moba_forward_varlen_lse on the same batch;
 *   workspace — at least moba_backward_workspace_size_varlen bytes (the
 *           largest one sequence needs), 256-byte aligned.
 * Every sequence is validated before anything is launched. */
moba_status_t moba_backward_workspace_size_varlen(const moba_problem_t* p, const int64_t* cu_seqlens,
                                        int64_t n_seqs, size_t* bytes);
moba_status_t moba_backward_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs,
                         const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const int32_t* block_idx, const float* lse, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Full causal softmax attention on the same layout, the method MoBA
 * approximates: with top_k covering every block MoBA becomes exactly this,
 * the switch to full attention [R] §1.2 describes for short inputs; MoBA's
 * speedup is measured against it ([P] §1 quotes the speedup over full
 * attention at 1M and 10M tokens).
 *   q, k, v — as for moba_forward (kv_heads honoured); o — output like q.
 * p->causal is ignored (always causal); block_size and top_k are
 * validated for sign only. Limits: head_dim in {64, 128}; any seq_len
 * below 2^27. Needs no workspace; errors as for moba_forward. */
moba_status_t moba_dense_causal_forward(const moba_problem_t* p, const void* q, const void* k,
                                        const void* v, void* o, void* stream);

/* moba_dense_causal_forward with the mask taken from p->causal (zero: full
 * non-causal attention, which MoBA equals when it keeps every block without
 * a causal mask). */
moba_status_t moba_dense_forward(const moba_problem_t* p, const void* q, const void* k, const void* v,
                                 void* o, void* stream);

/* Stage entry point (test/debug): the block summaries alone, step 1 of the
 * forward. Each block's keys are mean-pooled along the sequence ([P] §3.1,
 * gating score_fn mean_pool; [S] §3), or max / mean+max pooled per
 * p->pooling ([S] §3 names them as options).
 *   k    — device keys [batch, kv_heads, seq_len, head_dim];
 *   kbar — output, device float64 [batch, kv_heads, n_blocks, head_dim]:
 *          the pooled keys the gate scores against (a short last block
 *          pooled over the tokens it holds).
 * Uses the forward's workspace (moba_workspace_size). Errors as for
 * moba_forward, plus MOBA_ERR_NULL for a NULL kbar. */
moba_status_t moba_debug_pool(const moba_problem_t* p, const void* k, double* kbar, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Stage entry point (test/debug): pooling, the gate and the top-k choice
 * alone, steps 1-3 of the forward. Each query scores the eligible blocks by
 * its inner product with their pooled keys, future blocks masked ([P] §3.1
 * causal / mask_future), keeps its own block ([S] §3 force_current_block)
 * and the best top_k - 1 scored blocks, ties to the lower index (the
 * stable descending sort of [P] §4.1's routing check).
 *   q, k      — as for moba_forward;
 *   block_idx — output, exactly the block_idx moba_forward writes.
 * Uses the forward's workspace; errors as for moba_forward. */
moba_status_t moba_debug_gate_topk(const moba_problem_t* p, const void* q, const void* k, int32_t* block_idx,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Per-kernel timing with HIP events on the launching stream.
 * moba_timing_enable(1) creates an event pool (host call, not for use under
 * graph capture) and starts recording a begin/end event pair around every
 * kernel the library launches; moba_timing_enable(0) stops recording.
 * moba_timing_read synchronises on the recorded events, writes up to
 * max_entries {name, launches, total milliseconds} rows and clears the
 * record; *n_entries receives the number of kernels seen. */
typedef struct {
  const char* name;
  int64_t launches;
  double total_ms;
} moba_kernel_time_t;

moba_status_t moba_timing_enable(int enable);
moba_status_t moba_timing_read(moba_kernel_time_t* out, int max_entries, int* n_entries);

#ifdef __cplusplus
}
#endif
#endif /* MOBA_H */
