// C ABI of libmoba.so: validation, workspace layout and the launch sequence
// of the MoBA prefill forward (pool -> gate/top-k -> varlen pack -> past-block
// gather attention -> own-block attention + merge).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moba.h"
#include "launch.h"

namespace moba {

// ------------------------------------------------------------ errors
static thread_local std::string g_err;

static int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

// ------------------------------------------------------------ timing
namespace {
struct TimedLaunch {
  const char* name;
  hipEvent_t begin, end;
};
std::atomic<bool> g_timing{false};
std::mutex g_tmu;
std::vector<hipEvent_t> g_events;
std::vector<TimedLaunch> g_launches;
size_t g_next_event = 0;
constexpr size_t kEventPool = 2 * 16384;
}  // namespace

KernelTimer::KernelTimer(hipStream_t s, const char* name) : stream(s), slot(-1) {
  if (!g_timing.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_next_event + 2 > g_events.size()) return;
  TimedLaunch tl{name, g_events[g_next_event], g_events[g_next_event + 1]};
  g_next_event += 2;
  if (hipEventRecord(tl.begin, s) != hipSuccess) return;
  g_launches.push_back(tl);
  slot = (int)g_launches.size() - 1;
}

KernelTimer::~KernelTimer() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  (void)hipEventRecord(g_launches[slot].end, stream);
}

// ------------------------------------------------------------ planning
namespace {

constexpr size_t kAlign = 256;

// One launch chain: a batch of n_seq sequences, all of length S (uniform)
// or of the lengths in `lens` (a varlen batch), each with heads query heads
// and Hkv key/value heads.
struct Plan {
  int64_t B, H, S, D, Bs, top_k, bh, nb, k_eff, slots;  // S, nb, bh: the uniform batch's
  int64_t Hkv, G, bhkv;  // key/value heads, query heads per key/value head, B * Hkv
  bool causal, bf16_in, shared;
  int pooling;         // moba_pooling_t
  // the sequences
  bool uniform;
  int64_t n_seq, T, nb_total, max_nb, w128, w256, w1024;  // totals over the sequences
  std::vector<int64_t> tab;  // varlen: the sequence table (rows of kSeqCols prefix sums)
  int64_t pairs;       // (query, kept past block) pairs over all heads
  int64_t max_tiles;   // upper bound on gather tiles
  // workspace offsets (bytes)
  size_t kbar64, kbar32, kbar_hi, kbar_lo, norm, count, rank, offset, tile_start, qlist,
      tile_map, part_o, part_lse, seq_tab, total;
};

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Fields every problem shares; seq_len is checked by the caller.
int plan_common(const moba_problem_t* p, Plan* pl) {
  if (!p) return fail(MOBA_ERR_NULL, "problem pointer is NULL");
  const char* names[] = {"batch", "heads", "seq_len", "head_dim", "block_size"};
  const int64_t vals[] = {p->batch, p->heads, p->seq_len, p->head_dim, p->block_size};
  for (int i = 0; i < 5; ++i)
    if (vals[i] < 1) return fail(MOBA_ERR_SHAPE, std::string(names[i]) + " must be >= 1, got " + std::to_string(vals[i]));
  if (p->top_k < 1) return fail(MOBA_ERR_ARG, "top_k must be >= 1, got " + std::to_string(p->top_k));
  if (p->pooling != MOBA_POOL_MEAN && p->pooling != MOBA_POOL_MAX && p->pooling != MOBA_POOL_MEAN_MAX)
    return fail(MOBA_ERR_ARG, "pooling must be MOBA_POOL_MEAN (0), MOBA_POOL_MAX (1) or MOBA_POOL_MEAN_MAX (2), got " +
                                  std::to_string(p->pooling));
  if (p->reserved != 0) return fail(MOBA_ERR_ARG, "reserved must be 0, got " + std::to_string(p->reserved));
  if (p->reserved2 != 0) return fail(MOBA_ERR_ARG, "reserved2 must be 0, got " + std::to_string(p->reserved2));
  if (p->kv_heads < 0) return fail(MOBA_ERR_SHAPE, "kv_heads must be >= 0 (0 = heads), got " + std::to_string(p->kv_heads));
  if (p->kv_heads > 0 && p->heads % p->kv_heads != 0)
    return fail(MOBA_ERR_SHAPE, "heads (" + std::to_string(p->heads) + ") must be a multiple of kv_heads (" +
                                    std::to_string(p->kv_heads) + ")");
  if (p->dtype != MOBA_F32 && p->dtype != MOBA_BF16)
    return fail(MOBA_ERR_DTYPE, "dtype must be MOBA_F32 (0) or MOBA_BF16 (1), got " + std::to_string(p->dtype));
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(MOBA_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got " + std::to_string(p->head_dim));
  if (p->block_size % 64 != 0)
    return fail(MOBA_ERR_UNSUPPORTED, "block_size must be a multiple of 64, got " + std::to_string(p->block_size));
  Plan& P = *pl;
  P.B = p->batch;
  P.H = p->heads;
  P.D = p->head_dim;
  P.Bs = p->block_size;
  P.top_k = p->top_k;
  P.Hkv = p->kv_heads > 0 ? p->kv_heads : P.H;
  P.G = P.H / P.Hkv;
  P.bhkv = P.B * P.Hkv;
  P.bh = P.B * P.H;
  P.shared = p->gate_shared != 0;
  P.causal = p->causal != 0;
  P.bf16_in = p->dtype == MOBA_BF16;
  P.pooling = p->pooling;
  return MOBA_OK;
}

// (query, kept past block) pairs of one head of a sequence of len tokens.
int64_t head_pairs(const Plan& P, int64_t len) {
  const int64_t nb = (len + P.Bs - 1) / P.Bs;
  int64_t n = 0;
  for (int64_t c = 0; c < nb; ++c) {
    const int64_t elig = P.causal ? c : nb - 1;
    n += std::min(P.Bs, len - c * P.Bs) * std::min(P.slots, elig);
  }
  return n;
}

// The sequences: lens == nullptr for B sequences of S tokens (P.S set),
// else n lengths (a varlen batch). Sets totals, limits and the workspace.
int plan_seqs(Plan& P, const int64_t* lens, int64_t n, bool need_select, const char* what) {
  P.uniform = lens == nullptr;
  P.n_seq = n;
  auto len_of = [&](int64_t i) { return lens ? lens[i] : P.S; };
  P.T = P.nb_total = P.max_nb = P.w128 = P.w256 = P.w1024 = 0;
  if (!P.uniform) P.tab.assign((size_t)(n + 1) * kSeqCols, 0);
  for (int64_t i = 0; i <= n; ++i) {
    if (!P.uniform) {
      int64_t* row = &P.tab[(size_t)i * kSeqCols];
      row[kSeqTok] = P.T;
      row[kSeqBlk] = P.nb_total;
      row[kSeqW128] = P.w128;
      row[kSeqW256] = P.w256;
      row[kSeqW1024] = P.w1024;
    }
    if (i == n) break;
    const int64_t L = len_of(i);
    if (L >= (int64_t(1) << 27))
      return fail(MOBA_ERR_UNSUPPORTED, std::string(what) + " must be below 2^27, got " + std::to_string(L));
    const int64_t nbi = seq_units(kSeqBlk, L, P.Bs);
    P.T += L;
    P.nb_total += nbi;
    P.max_nb = std::max(P.max_nb, nbi);
    P.w128 += seq_units(kSeqW128, L, P.Bs);
    P.w256 += seq_units(kSeqW256, L, P.Bs);
    P.w1024 += seq_units(kSeqW1024, L, P.Bs);
    if (P.uniform) break;  // every sequence alike: scale below
  }
  if (P.uniform) {
    P.T *= n;
    P.nb = P.nb_total;
    P.nb_total *= n;
    P.w128 *= n;
    P.w256 *= n;
    P.w1024 *= n;
  }
  // k_eff - 1 past-block slots per query row: a sequence with fewer blocks
  // keeps min(top_k - 1, eligible) <= its own count of them.
  P.k_eff = std::min(P.top_k, P.max_nb);
  P.slots = P.k_eff - 1;
  if (P.H * P.nb_total >= (int64_t(1) << 31))
    return fail(MOBA_ERR_UNSUPPORTED, "heads * blocks (over all sequences) must be below 2^31");
  for (int64_t i = 0; i < n; ++i) {
    const int64_t nbi = seq_units(kSeqBlk, len_of(i), P.Bs);
    const int64_t si = std::min(P.top_k, nbi) - 1;
    if (si > kMaxSlotsHost && P.top_k < nbi)
      return fail(MOBA_ERR_UNSUPPORTED, "top_k " + std::to_string(P.top_k) + " keeps more than " +
                                            std::to_string(kMaxSlotsHost) + " past blocks per query; use top_k <= " +
                                            std::to_string(kMaxSlotsHost + 1) + " or top_k >= n_blocks (" +
                                            std::to_string(nbi) + ")");
    if (P.uniform) break;
  }
  if (P.H * P.T * std::max<int64_t>(P.slots, 1) >= (int64_t(1) << 31))
    return fail(MOBA_ERR_UNSUPPORTED,
                "heads * tokens * (min(top_k, n_blocks) - 1) must be below 2^31 (int32 list entries)");
  // Exact pair count: every query in block c keeps min(k_eff - 1, eligible) past blocks.
  P.pairs = 0;
  if (P.uniform) {
    P.pairs = head_pairs(P, P.S) * P.H * n;
  } else {
    for (int64_t i = 0; i < n; ++i) P.pairs += head_pairs(P, lens[i]) * P.H;
  }
  if (P.pairs >= (int64_t(1) << 31)) return fail(MOBA_ERR_UNSUPPORTED, "too many (query, block) pairs for int32 lists");
  P.max_tiles = P.pairs / kGatherTileM + P.H * P.nb_total + 1;
  const size_t esz = P.bf16_in ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up(bytes);
    return at;
  };
  // Block summaries per key/value head; counts per query head.
  const size_t kvb = (size_t)(P.Hkv * P.nb_total), qb = (size_t)(P.H * P.nb_total);
  const size_t rows = (size_t)(P.H * P.T);
  P.kbar64 = take(kvb * P.D * 8);
  P.kbar32 = take(kvb * P.D * 4);
  P.kbar_hi = take(kvb * P.D * 2);
  P.kbar_lo = take(kvb * P.D * 2);
  P.norm = take(kvb * 4);
  P.count = take(qb * 4);
  P.rank = take(rows * P.slots * 4);
  P.seq_tab = P.uniform ? 0 : take(P.tab.size() * 8);
  if (need_select) {
    P.offset = take((qb + 1) * 4);
    P.tile_start = take((qb + 1) * 4);
    P.qlist = take((size_t)P.pairs * 4);
    P.tile_map = take((size_t)gather_grid_for(P.max_tiles) * 16);
    P.part_o = take(rows * P.slots * P.D * esz);
    P.part_lse = take(rows * P.slots * 4);
  }
  P.total = off;
  return MOBA_OK;
}

// A batch of equal-length sequences ([batch, heads, seq_len, head_dim]).
int plan_problem(const moba_problem_t* p, Plan* pl, bool need_select) {
  int st = plan_common(p, pl);
  if (st != MOBA_OK) return st;
  pl->S = p->seq_len;
  return plan_seqs(*pl, nullptr, p->batch, need_select, "seq_len");
}

Seqs seqs_of(const Plan& P, void* ws) {
  Seqs q;
  q.tab = P.uniform ? nullptr : reinterpret_cast<const int64_t*>(static_cast<char*>(ws) + P.seq_tab);
  q.n = P.n_seq;
  q.len = P.uniform ? P.S : 0;
  return q;
}

// Backward workspace: the forward's plan (its lists and tiles are rebuilt
// from block_idx) plus delta and the log2-domain log-sum-exp per query, the
// past-block dq partials, all fp32, the ordered ranks' chunk counts, and per
// list position its query row, log-sum-exp and delta.
struct BwdPlan {
  size_t delta, lse2, dq_part, chunk_counts, lt, ll, ld, total;
};
BwdPlan plan_backward(const Plan& P) {
  BwdPlan B;
  size_t off = P.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up(bytes);
    return at;
  };
  const size_t rows = (size_t)(P.bh * P.S);
  B.delta = take(rows * 4);
  B.lse2 = take(rows * 4);
  B.dq_part = take(rows * (size_t)P.slots * (size_t)P.D * 2);
  B.chunk_counts = take((size_t)P.bh * (size_t)((P.S + rank_chunk(P.S) - 1) / rank_chunk(P.S)) * (size_t)P.nb * 4);
  B.lt = take((size_t)P.pairs * 4);
  B.ll = take((size_t)P.pairs * 4);
  B.ld = take((size_t)P.pairs * 4);
  B.total = off;
  return B;
}

int check_ws(const Plan& P, void* ws, size_t bytes) {
  if (bytes < P.total)
    return fail(MOBA_ERR_WORKSPACE, "workspace_bytes " + std::to_string(bytes) + " < required " + std::to_string(P.total));
  if (P.total > 0 && !ws) return fail(MOBA_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return fail(MOBA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return MOBA_OK;
}

int dev_fail(hipError_t e, const char* what) {
  return fail(MOBA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

#define MOBA_TRY(expr, what)                     \
  do {                                           \
    hipError_t _e = (expr);                      \
    if (_e != hipSuccess) return dev_fail(_e, what); \
  } while (0)

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// pool + gate: writes block_idx, counts and ranks.
int run_select(const Plan& P, const void* q, const void* k, int32_t* block_idx, void* ws, hipStream_t s,
               double* kbar64_out) {
  const Seqs sq = seqs_of(P, ws);
  if (!P.uniform)
    MOBA_TRY(hipMemcpyAsync(static_cast<char*>(ws) + P.seq_tab, P.tab.data(), P.tab.size() * sizeof(int64_t),
                            hipMemcpyHostToDevice, s),
             "sequence table copy");
  PoolArgs pa{};
  pa.k = k;
  pa.sq = sq;
  pa.kv_heads = P.Hkv;
  pa.kv_blocks = P.Hkv * P.nb_total;
  pa.group = (int)P.G;
  pa.block_size = P.Bs;
  pa.head_dim = (int)P.D;
  pa.bf16_in = P.bf16_in;
  pa.pooling = P.pooling;
  pa.kbar64 = kbar64_out ? kbar64_out : at<double>(ws, P.kbar64);
  pa.kbar32 = at<float>(ws, P.kbar32);
  pa.kbar_hi = at<bf16>(ws, P.kbar_hi);
  pa.kbar_lo = at<bf16>(ws, P.kbar_lo);
  pa.norm = at<float>(ws, P.norm);
  pa.count = at<int32_t>(ws, P.count);
  MOBA_TRY(launch_pool(pa, s), "pool launch");
  if (!block_idx) return MOBA_OK;
  GateArgs ga{};
  ga.q = q;
  ga.kbar64 = pa.kbar64;
  ga.kbar32 = pa.kbar32;
  ga.kbar_hi = pa.kbar_hi;
  ga.kbar_lo = pa.kbar_lo;
  ga.norm = pa.norm;
  ga.sq = sq;
  ga.heads = P.H;
  ga.kv_heads = P.Hkv;
  ga.block_size = P.Bs;
  ga.max_nb = P.max_nb;
  ga.gate_wgs = (P.shared && P.G > 1 ? P.Hkv : P.H) * P.w128;
  ga.gate_wgs256 = P.H * P.w256;
  ga.rank_wgs = P.H * P.w1024;
  ga.head_dim = (int)P.D;
  ga.bf16_in = P.bf16_in;
  ga.causal = P.causal;
  ga.top_k = (int)P.top_k;
  ga.k_eff = (int)P.k_eff;
  ga.block_idx = block_idx;
  ga.count = at<int32_t>(ws, P.count);
  ga.rank = at<int32_t>(ws, P.rank);
  ga.group = (int)P.G;
  ga.shared = P.shared;
  MOBA_TRY(launch_gate(ga, s), "gate launch");
  return MOBA_OK;
}

AttnArgs attn_args(const Plan& P, const void* q, const void* k, const void* v, void* o, void* ws) {
  AttnArgs aa{};
  aa.q = q;
  aa.k = k;
  aa.v = v;
  aa.o = o;
  aa.sq = seqs_of(P, ws);
  aa.heads = P.H;
  aa.block_size = P.Bs;
  aa.diag_wgs = P.H * P.w128;
  aa.head_dim = (int)P.D;
  aa.bf16_in = P.bf16_in;
  aa.causal = P.causal;
  aa.k_eff = (int)P.k_eff;
  aa.group = (int)P.G;
  return aa;
}

PackArgs pack_args(const Plan& P, const int32_t* block_idx, void* ws) {
  PackArgs pk{};
  pk.sq = seqs_of(P, ws);
  pk.heads = P.H;
  pk.block_size = P.Bs;
  pk.rows = P.H * P.T;
  pk.q_blocks = P.H * P.nb_total;
  pk.causal = P.causal;
  pk.top_k = (int)P.top_k;
  pk.k_eff = (int)P.k_eff;
  pk.tile_m = kGatherTileM;
  pk.block_idx = block_idx;
  pk.count = at<int32_t>(ws, P.count);
  pk.rank = at<int32_t>(ws, P.rank);
  pk.offset = at<int32_t>(ws, P.offset);
  pk.tile_start = at<int32_t>(ws, P.tile_start);
  pk.qlist = at<int32_t>(ws, P.qlist);
  pk.grid = gather_grid_for(P.max_tiles);
  pk.tile_map = at<int32_t>(ws, P.tile_map);
  return pk;
}

}  // namespace
}  // namespace moba

using namespace moba;

namespace {
int check_tensors(const void* q, const void* k, const void* v, const void* o, const int32_t* block_idx) {
  if (!q) return fail(MOBA_ERR_NULL, "q is NULL");
  if (!k) return fail(MOBA_ERR_NULL, "k is NULL");
  if (!v) return fail(MOBA_ERR_NULL, "v is NULL");
  if (!o) return fail(MOBA_ERR_NULL, "o is NULL");
  if (!block_idx) return fail(MOBA_ERR_NULL, "block_idx is NULL");
  return MOBA_OK;
}

// The whole forward of one validated problem, queued on s.
int run_forward(const Plan& P, const void* q, const void* k, const void* v, void* o, int32_t* block_idx,
                void* workspace, hipStream_t s, float* lse = nullptr) {
  int st = run_select(P, q, k, block_idx, workspace, s, nullptr);
  if (st != MOBA_OK) return st;
  AttnArgs aa = attn_args(P, q, k, v, o, workspace);
  aa.lse_out = lse;
  aa.part_o = at<void>(workspace, P.part_o);
  aa.part_lse = at<float>(workspace, P.part_lse);
  if (P.pairs > 0) {
    const PackArgs pk = pack_args(P, block_idx, workspace);
    MOBA_TRY(launch_pack(pk, s), "pack launch");
    aa.qlist = pk.qlist;
    aa.tile_map = pk.tile_map;
    aa.gather_grid = pk.grid;
    MOBA_TRY(launch_gather(aa, s), "gather launch");
  }
  MOBA_TRY(launch_diag_merge(aa, s), "diag launch");
  return MOBA_OK;
}

// A varlen batch: n sequences of the cu_seqlens lengths, one plan (and one
// launch chain) for all of them.
int varlen_plan(const moba_problem_t* p, const int64_t* cu, int64_t n, Plan* P) {
  if (!p) return fail(MOBA_ERR_NULL, "problem pointer is NULL");
  if (!cu) return fail(MOBA_ERR_NULL, "cu_seqlens is NULL");
  if (n < 1) return fail(MOBA_ERR_ARG, "n_seqs must be >= 1, got " + std::to_string(n));
  if (cu[0] != 0) return fail(MOBA_ERR_ARG, "cu_seqlens[0] must be 0, got " + std::to_string(cu[0]));
  if (p->batch != n)
    return fail(MOBA_ERR_ARG, "batch must equal n_seqs (" + std::to_string(n) + "), got " + std::to_string(p->batch));
  if (p->seq_len != cu[n])
    return fail(MOBA_ERR_ARG, "seq_len must equal cu_seqlens[n_seqs] (" + std::to_string(cu[n]) + "), got " +
                                  std::to_string(p->seq_len));
  std::vector<int64_t> lens((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    lens[(size_t)i] = cu[i + 1] - cu[i];
    if (lens[(size_t)i] < 1)
      return fail(MOBA_ERR_SHAPE, "sequence " + std::to_string(i) + " has length " + std::to_string(lens[(size_t)i]) +
                                      " (cu_seqlens must increase)");
  }
  int st = plan_common(p, P);
  if (st != MOBA_OK) return st;
  P->S = 0;
  return plan_seqs(*P, lens.data(), n, true, "every sequence length");
}
}  // namespace

namespace {

const char* status_text(int status) {
  switch (status) {
    case MOBA_OK: return "ok";
    case MOBA_ERR_NULL: return "null pointer";
    case MOBA_ERR_SHAPE: return "invalid shape";
    case MOBA_ERR_ARG: return "invalid argument";
    case MOBA_ERR_DTYPE: return "invalid dtype";
    case MOBA_ERR_UNSUPPORTED: return "outside kernel limits";
    case MOBA_ERR_WORKSPACE: return "workspace too small";
    case MOBA_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

int impl_workspace_size(const moba_problem_t* p, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MOBA_ERR_NULL, "bytes pointer is NULL");
  Plan P;
  const int st = plan_problem(p, &P, true);
  if (st != MOBA_OK) return st;
  *bytes = P.total;
  return MOBA_OK;
}

int impl_forward(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                 int32_t* block_idx, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  Plan P;
  int st = plan_problem(p, &P, true);
  if (st != MOBA_OK) return st;
  st = check_tensors(q, k, v, o, block_idx);
  if (st != MOBA_OK) return st;
  st = check_ws(P, workspace, workspace_bytes);
  if (st != MOBA_OK) return st;
  return run_forward(P, q, k, v, o, block_idx, workspace, static_cast<hipStream_t>(stream));
}

int impl_forward_lse(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                     int32_t* block_idx, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  Plan P;
  int st = plan_problem(p, &P, true);
  if (st != MOBA_OK) return st;
  st = check_tensors(q, k, v, o, block_idx);
  if (st != MOBA_OK) return st;
  if (!lse) return fail(MOBA_ERR_NULL, "lse is NULL");
  st = check_ws(P, workspace, workspace_bytes);
  if (st != MOBA_OK) return st;
  return run_forward(P, q, k, v, o, block_idx, workspace, static_cast<hipStream_t>(stream), lse);
}

int plan_backward_problem(const moba_problem_t* p, Plan* P, BwdPlan* B) {
  const int st = plan_problem(p, P, true);
  if (st != MOBA_OK) return st;
  if (!P->bf16_in) return fail(MOBA_ERR_UNSUPPORTED, "the backward supports bf16 inputs only (dtype MOBA_BF16)");
  if (P->nb > 16384) return fail(MOBA_ERR_UNSUPPORTED, "the backward supports at most 16384 blocks");
  *B = plan_backward(*P);
  return MOBA_OK;
}

int impl_backward_workspace_size(const moba_problem_t* p, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MOBA_ERR_NULL, "bytes pointer is NULL");
  Plan P;
  BwdPlan B;
  const int st = plan_backward_problem(p, &P, &B);
  if (st != MOBA_OK) return st;
  *bytes = B.total;
  return MOBA_OK;
}

// The backward's pointers and workspace, checked once every problem is valid.
int check_backward_buffers(const void* const (&ins)[10], size_t need, const void* workspace,
                           size_t workspace_bytes) {
  const char* names[] = {"q", "k", "v", "o", "dout", "block_idx", "lse", "dq", "dk", "dv"};
  for (int i = 0; i < 10; ++i)
    if (!ins[i]) return fail(MOBA_ERR_NULL, std::string(names[i]) + " is NULL");
  if (workspace_bytes < need)
    return fail(MOBA_ERR_WORKSPACE, "workspace_bytes " + std::to_string(workspace_bytes) + " < required " +
                                        std::to_string(need));
  if (!workspace) return fail(MOBA_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(MOBA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return MOBA_OK;
}

// The whole backward of one validated (uniform) problem, queued on s.
int run_backward(const Plan& P, const BwdPlan& B, const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const int32_t* block_idx, const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, hipStream_t s) {
  BwdArgs ba{};
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.o = o;
  ba.dout = dout;
  ba.lse = lse;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.bh = P.bh;
  ba.seq_len = P.S;
  ba.block_size = P.Bs;
  ba.n_blocks = P.nb;
  ba.head_dim = (int)P.D;
  ba.causal = P.causal;
  ba.k_eff = (int)P.k_eff;
  ba.group = (int)P.G;
  ba.block_idx = block_idx;
  ba.top_k = (int)P.top_k;
  ba.delta = at<float>(workspace, B.delta);
  ba.lse2 = at<float>(workspace, B.lse2);
  ba.dq_part = at<bf16>(workspace, B.dq_part);
  ba.lt = at<int32_t>(workspace, B.lt);
  ba.ll = at<float>(workspace, B.ll);
  ba.ld = at<float>(workspace, B.ld);
  if (P.pairs > 0) {
    // The forward's varlen lists, rebuilt from block_idx in a fixed order
    // (dk and dv sum over them): counts, ranks, offsets, lists, tiles.
    int32_t* count = at<int32_t>(workspace, P.count);
    GateArgs ga{};
    ga.bh = P.bh;
    ga.seq_len = P.S;
    ga.block_size = P.Bs;
    ga.n_blocks = P.nb;
    ga.causal = P.causal;
    ga.top_k = (int)P.top_k;
    ga.k_eff = (int)P.k_eff;
    ga.block_idx = const_cast<int32_t*>(block_idx);
    ga.count = count;
    ga.rank = at<int32_t>(workspace, P.rank);
    ga.group = (int)P.G;
    MOBA_TRY(launch_rank(ga, s, at<int32_t>(workspace, B.chunk_counts)), "rank launch");
    const PackArgs pk = pack_args(P, block_idx, workspace);
    MOBA_TRY(launch_pack(pk, s), "pack launch");
    ba.qlist = pk.qlist;
    ba.offset = pk.offset;
    ba.tile_map = pk.tile_map;
    ba.gather_grid = pk.grid;
  }
  MOBA_TRY(launch_backward(ba, s), "backward launch");
  return MOBA_OK;
}

int impl_backward(const moba_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const int32_t* block_idx, const float* lse, void* dq, void* dk, void* dv,
                  void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  Plan P;
  BwdPlan B;
  int st = plan_backward_problem(p, &P, &B);
  if (st != MOBA_OK) return st;
  st = check_backward_buffers({q, k, v, o, dout, block_idx, lse, dq, dk, dv}, B.total, workspace, workspace_bytes);
  if (st != MOBA_OK) return st;
  return run_backward(P, B, q, k, v, o, dout, block_idx, lse, dq, dk, dv, workspace,
                      static_cast<hipStream_t>(stream));
}

// A varlen batch's backward: every sequence planned as its own uniform
// problem (batch 1, seq_len len_i); the workspace is the largest of theirs.
int plan_backward_varlen(const moba_problem_t* p, const int64_t* cu, int64_t n, std::vector<Plan>* Ps,
                         std::vector<BwdPlan>* Bs, size_t* need) {
  Plan V;
  int st = varlen_plan(p, cu, n, &V);  // lengths, batch and seq_len against cu_seqlens
  if (st != MOBA_OK) return st;
  Ps->assign((size_t)n, Plan{});
  Bs->assign((size_t)n, BwdPlan{});
  *need = 0;
  for (int64_t i = 0; i < n; ++i) {
    moba_problem_t one = *p;
    one.batch = 1;
    one.seq_len = cu[i + 1] - cu[i];
    st = plan_backward_problem(&one, &(*Ps)[(size_t)i], &(*Bs)[(size_t)i]);
    if (st != MOBA_OK) return fail(st, "sequence " + std::to_string(i) + ": " + g_err);
    *need = std::max(*need, (*Bs)[(size_t)i].total);
  }
  return MOBA_OK;
}

int impl_backward_workspace_size_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs,
                                        size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MOBA_ERR_NULL, "bytes pointer is NULL");
  std::vector<Plan> Ps;
  std::vector<BwdPlan> Bs;
  return plan_backward_varlen(p, cu_seqlens, n_seqs, &Ps, &Bs, bytes);
}

int impl_backward_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs, const void* q,
                         const void* k, const void* v, const void* o, const void* dout, const int32_t* block_idx,
                         const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_err.clear();
  std::vector<Plan> Ps;
  std::vector<BwdPlan> Bs;
  size_t need = 0;
  int st = plan_backward_varlen(p, cu_seqlens, n_seqs, &Ps, &Bs, &need);
  if (st != MOBA_OK) return st;
  st = check_backward_buffers({q, k, v, o, dout, block_idx, lse, dq, dk, dv}, need, workspace, workspace_bytes);
  if (st != MOBA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // Sequence i is a uniform [1, heads, len_i, D] problem from token
  // cu_seqlens[i]; the sequences run one after another on the stream and
  // reuse the workspace (bf16 inputs: 2 bytes per element).
  const int64_t H = p->heads, Hkv = Ps[0].Hkv, D = p->head_dim, K = p->top_k;
  for (int64_t i = 0; i < n_seqs; ++i) {
    const int64_t t0 = cu_seqlens[i];
    const size_t qoff = (size_t)(t0 * H * D * 2), kvoff = (size_t)(t0 * Hkv * D * 2);
    auto in = [](const void* x, size_t off) { return static_cast<const char*>(x) + off; };
    auto out = [](void* x, size_t off) { return static_cast<char*>(x) + off; };
    st = run_backward(Ps[(size_t)i], Bs[(size_t)i], in(q, qoff), in(k, kvoff), in(v, kvoff), in(o, qoff),
                      in(dout, qoff), block_idx + t0 * H * K, lse + t0 * H, out(dq, qoff), out(dk, kvoff),
                      out(dv, kvoff), workspace, s);
    if (st != MOBA_OK) return st;
  }
  return MOBA_OK;
}

int impl_workspace_size_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MOBA_ERR_NULL, "bytes pointer is NULL");
  Plan P;
  const int st = varlen_plan(p, cu_seqlens, n_seqs, &P);
  if (st != MOBA_OK) return st;
  *bytes = P.total;
  return MOBA_OK;
}

int impl_forward_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs, const void* q,
                        const void* k, const void* v, void* o, int32_t* block_idx, void* workspace,
                        size_t workspace_bytes, void* stream, float* lse = nullptr, bool want_lse = false) {
  g_err.clear();
  Plan P;
  int st = varlen_plan(p, cu_seqlens, n_seqs, &P);
  if (st != MOBA_OK) return st;
  st = check_tensors(q, k, v, o, block_idx);
  if (st != MOBA_OK) return st;
  if (want_lse && !lse) return fail(MOBA_ERR_NULL, "lse is NULL");
  st = check_ws(P, workspace, workspace_bytes);
  if (st != MOBA_OK) return st;
  // Every sequence is validated above; one launch chain covers them all.
  return run_forward(P, q, k, v, o, block_idx, workspace, static_cast<hipStream_t>(stream), lse);
}

int impl_dense_forward(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                       void* stream, bool force_causal) {
  g_err.clear();
  if (!p) return fail(MOBA_ERR_NULL, "problem pointer is NULL");
  // Dense attention ignores the block structure: validate it as a problem
  // whose only block is the whole sequence.
  moba_problem_t d = *p;
  if (force_causal) d.causal = 1;
  d.block_size = 64;
  if (d.top_k < 1) return fail(MOBA_ERR_ARG, "top_k must be >= 1, got " + std::to_string(p->top_k));
  if (p->block_size < 1) return fail(MOBA_ERR_SHAPE, "block_size must be >= 1, got " + std::to_string(p->block_size));
  d.top_k = 1;
  Plan P;
  const int st = plan_problem(&d, &P, false);
  if (st != MOBA_OK) return st;
  if (!q) return fail(MOBA_ERR_NULL, "q is NULL");
  if (!k) return fail(MOBA_ERR_NULL, "k is NULL");
  if (!v) return fail(MOBA_ERR_NULL, "v is NULL");
  if (!o) return fail(MOBA_ERR_NULL, "o is NULL");
  AttnArgs aa = attn_args(P, q, k, v, o, nullptr);
  MOBA_TRY(launch_dense(aa, static_cast<hipStream_t>(stream)), "dense launch");
  return MOBA_OK;
}

int impl_pool(const moba_problem_t* p, const void* k, double* kbar, void* workspace, size_t workspace_bytes,
              void* stream) {
  g_err.clear();
  Plan P;
  int st = plan_problem(p, &P, true);
  if (st != MOBA_OK) return st;
  if (!k) return fail(MOBA_ERR_NULL, "k is NULL");
  if (!kbar) return fail(MOBA_ERR_NULL, "kbar is NULL");
  st = check_ws(P, workspace, workspace_bytes);
  if (st != MOBA_OK) return st;
  return run_select(P, nullptr, k, nullptr, workspace, static_cast<hipStream_t>(stream), kbar);
}

int impl_select(const moba_problem_t* p, const void* q, const void* k, int32_t* block_idx, void* workspace,
                size_t workspace_bytes, void* stream) {
  g_err.clear();
  Plan P;
  int st = plan_problem(p, &P, true);
  if (st != MOBA_OK) return st;
  if (!q) return fail(MOBA_ERR_NULL, "q is NULL");
  if (!k) return fail(MOBA_ERR_NULL, "k is NULL");
  if (!block_idx) return fail(MOBA_ERR_NULL, "block_idx is NULL");
  st = check_ws(P, workspace, workspace_bytes);
  if (st != MOBA_OK) return st;
  return run_select(P, q, k, block_idx, workspace, static_cast<hipStream_t>(stream), nullptr);
}

int impl_timing_enable(int enable) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_tmu);
  if (enable && g_events.empty()) {
    g_events.resize(kEventPool);
    for (auto& e : g_events) {
      const hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) {
        g_events.clear();
        return dev_fail(r, "hipEventCreate");
      }
    }
  }
  g_timing.store(enable != 0);
  return MOBA_OK;
}

int impl_timing_read(moba_kernel_time_t* out, int max_entries, int* n_entries) {
  g_err.clear();
  if (!n_entries) return fail(MOBA_ERR_NULL, "n_entries is NULL");
  std::lock_guard<std::mutex> lk(g_tmu);
  std::vector<moba_kernel_time_t> agg;
  for (const auto& tl : g_launches) {
    hipError_t r = hipEventSynchronize(tl.end);
    if (r != hipSuccess) return dev_fail(r, "hipEventSynchronize");
    float ms = 0.f;
    r = hipEventElapsedTime(&ms, tl.begin, tl.end);
    if (r != hipSuccess) return dev_fail(r, "hipEventElapsedTime");
    auto it = std::find_if(agg.begin(), agg.end(),
                           [&](const moba_kernel_time_t& x) { return std::strcmp(x.name, tl.name) == 0; });
    if (it == agg.end()) agg.push_back({tl.name, 1, (double)ms});
    else {
      it->launches += 1;
      it->total_ms += ms;
    }
  }
  g_launches.clear();
  g_next_event = 0;
  *n_entries = (int)agg.size();
  for (int i = 0; i < (int)agg.size() && i < max_entries; ++i) out[i] = agg[i];
  return MOBA_OK;
}

}  // namespace

// ------------------------------------------------ allocation-free forward
// The workspace of moba_forward_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends. In host code `scratch` only
// names the symbol; its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept, and only that
// address is passed to kernels.
static __device__ __align__(256) char scratch[MOBA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device ordinal; nullptr until looked up

int scratch_on_current_device(void** out) {
  int dev = -1;
  MOBA_TRY(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev >= (int)g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[(size_t)dev]) {
    void* ptr = nullptr;
    MOBA_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % kAlign != 0)
      return fail(MOBA_ERR_DEVICE, "the scratch array's device address is NULL or not 256-byte aligned");
    g_scratch_ptr[(size_t)dev] = ptr;
  }
  *out = g_scratch_ptr[(size_t)dev];
  return MOBA_OK;
}

int impl_forward_noalloc(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                         int32_t* block_idx, void* stream) {
  g_err.clear();
  Plan P;
  int st = plan_problem(p, &P, true);
  if (st != MOBA_OK) return st;
  st = check_tensors(q, k, v, o, block_idx);
  if (st != MOBA_OK) return st;
  if (P.total > (size_t)MOBA_NOALLOC_SCRATCH_BYTES)
    return fail(MOBA_ERR_WORKSPACE, "problem needs " + std::to_string(P.total) +
                                        " bytes of scratch, above the " +
                                        std::to_string((size_t)MOBA_NOALLOC_SCRATCH_BYTES) +
                                        " bytes moba_forward_noalloc holds per GPU; use moba_forward with a "
                                        "caller-allocated workspace");
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != MOBA_OK) return st;
  // Nothing in the scratch needs clearing: the forward never reads a byte
  // of its workspace before writing it (the pool kernel zeroes the block
  // counts the gate's ranking then fills).
  return run_forward(P, q, k, v, o, block_idx, ws, static_cast<hipStream_t>(stream));
}
}  // namespace

// ------------------------------------------------------------ the C ABI
extern "C" {

static inline moba_status_t st_(int s) { return static_cast<moba_status_t>(s); }

int moba_abi_version(void) { return MOBA_ABI_VERSION; }

const char* moba_status_str(moba_status_t status) { return status_text(static_cast<int>(status)); }

const char* moba_last_error(void) { return g_err.c_str(); }

moba_status_t moba_workspace_size(const moba_problem_t* p, size_t* bytes) { return st_(impl_workspace_size(p, bytes)); }

moba_status_t moba_forward(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                           int32_t* block_idx, void* workspace, size_t workspace_bytes, void* stream) {
  return st_(impl_forward(p, q, k, v, o, block_idx, workspace, workspace_bytes, stream));
}

moba_status_t moba_forward_noalloc(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                                   int32_t* block_idx, void* stream) {
  return st_(impl_forward_noalloc(p, q, k, v, o, block_idx, stream));
}

moba_status_t moba_forward_lse(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                               int32_t* block_idx, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return st_(impl_forward_lse(p, q, k, v, o, block_idx, lse, workspace, workspace_bytes, stream));
}

moba_status_t moba_backward_workspace_size(const moba_problem_t* p, size_t* bytes) {
  return st_(impl_backward_workspace_size(p, bytes));
}

moba_status_t moba_backward(const moba_problem_t* p, const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const int32_t* block_idx, const float* lse, void* dq, void* dk,
                            void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return st_(impl_backward(p, q, k, v, o, dout, block_idx, lse, dq, dk, dv, workspace, workspace_bytes, stream));
}

moba_status_t moba_workspace_size_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs,
                                         size_t* bytes) {
  return st_(impl_workspace_size_varlen(p, cu_seqlens, n_seqs, bytes));
}

moba_status_t moba_forward_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs,
                                  const void* q, const void* k, const void* v, void* o, int32_t* block_idx,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return st_(impl_forward_varlen(p, cu_seqlens, n_seqs, q, k, v, o, block_idx, workspace, workspace_bytes, stream));
}

moba_status_t moba_forward_varlen_lse(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs,
                                      const void* q, const void* k, const void* v, void* o, int32_t* block_idx,
                                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return st_(impl_forward_varlen(p, cu_seqlens, n_seqs, q, k, v, o, block_idx, workspace, workspace_bytes, stream,
                                 lse, true));
}

moba_status_t moba_backward_workspace_size_varlen(const moba_problem_t* p, const int64_t* cu_seqlens,
                                                  int64_t n_seqs, size_t* bytes) {
  return st_(impl_backward_workspace_size_varlen(p, cu_seqlens, n_seqs, bytes));
}

moba_status_t moba_backward_varlen(const moba_problem_t* p, const int64_t* cu_seqlens, int64_t n_seqs,
                                   const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const int32_t* block_idx, const float* lse, void* dq, void* dk, void* dv,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return st_(impl_backward_varlen(p, cu_seqlens, n_seqs, q, k, v, o, dout, block_idx, lse, dq, dk, dv, workspace,
                                  workspace_bytes, stream));
}

moba_status_t moba_dense_causal_forward(const moba_problem_t* p, const void* q, const void* k, const void* v,
                                        void* o, void* stream) {
  return st_(impl_dense_forward(p, q, k, v, o, stream, true));
}

moba_status_t moba_dense_forward(const moba_problem_t* p, const void* q, const void* k, const void* v, void* o,
                                 void* stream) {
  return st_(impl_dense_forward(p, q, k, v, o, stream, false));
}

moba_status_t moba_debug_pool(const moba_problem_t* p, const void* k, double* kbar, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return st_(impl_pool(p, k, kbar, workspace, workspace_bytes, stream));
}

moba_status_t moba_debug_gate_topk(const moba_problem_t* p, const void* q, const void* k, int32_t* block_idx,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return st_(impl_select(p, q, k, block_idx, workspace, workspace_bytes, stream));
}

moba_status_t moba_timing_enable(int enable) { return st_(impl_timing_enable(enable)); }

moba_status_t moba_timing_read(moba_kernel_time_t* out, int max_entries, int* n_entries) {
  return st_(impl_timing_read(out, max_entries, n_entries));
}

}  // extern "C"
