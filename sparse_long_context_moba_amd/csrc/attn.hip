// Attention over the routed blocks, on MFMA with an online softmax.
//
// MoBA attends only the keys of the blocks a query kept, with the causal
// mask inside the query's own block, and normalises once over the union of
// those keys («MoBA 复现代码跑不通…» §3.3; the hncyxsy.com MOBA article §3).
// The union is split into two disjoint parts that are merged exactly:
//
//  gather_attn  — past blocks. Work is grouped by key block: a workgroup
//                 takes up to 128 queries from one block's varlen list,
//                 streams that block's K/V through LDS in 64-key subtiles and
//                 writes, per (query, slot), the normalised partial output
//                 and its log2-sum-exp.
//  diag_merge   — the own block. A workgroup takes 128 consecutive queries
//                 (32 per wave; a wave's queries share one block, which is a
//                 multiple of 64 long, while a workgroup's may span two or
//                 more blocks), starts each query's online softmax from its
//                 past partials (the log-sum-exp merge, done first), attends
//                 its block's keys up to the query (causal) and writes o in
//                 the input dtype.
//  dense_attn   — plain full attention (causal or not) with the same engine,
//                 the baseline MoBA is measured against.
//
// Engine (one wave = 32 queries): S^T = K Q^T on MFMA 32x32x16 bf16 (K from
// LDS as the A operand, Q held in registers as the B operand), so lane l
// holds 32 scores of query l%32 per 64 keys and the row statistics need a
// single exchange with lane l^32. P stays in registers and feeds
// O^T = V^T P^T directly as the B operand.
// bf16 K/V subtiles move HBM -> LDS by direct loads (global_load_lds, 16 B
// per lane, double-buffered, no register staging) into a row-major layout
// whose 16-byte chunks are XOR-swizzled per row. The A operand of P.V is
// read with the LDS transpose load ds_read_b64_tr_b16: 16 lanes naming a
// 4-key x 16-dim patch of V receive V^T fragments directly. Separate
// swizzles for K and V keep the K reads (16 rows at one chunk) and the
// transpose reads (4 rows x 4 chunks per 32 lanes) free of bank conflicts.
// fp32 inputs use MFMA 32x32x2 f32 with the same register layout and
// register-staged LDS tiles.
#include <algorithm>

#include "engine.h"

namespace moba {

// Waves per SIMD the register budget is set for: two, except fp32 inputs
// at head_dim 128, whose query fragment (64 registers) and staged K/V
// subtile (64) beside the output accumulators (64) do not fit in 256
// registers; they run at one wave per SIMD with the whole register file.
template <typename T, int D>
constexpr int attn_waves() {
  return sizeof(T) == 4 && D == 128 ? 1 : 2;
}

// ------------------------------------------------------- past-block gather
template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(attn_waves<T, D>()))) void
gather_attn_kernel(AttnArgs a) {
  using E = typename EngOf<T, D>::type;
  constexpr int NT = 64 * NW;
  MOBA_KERNEL_LDS(E)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;

  // This workgroup's tile: its block, list range and sequence (written by
  // the packing step, which also spreads tiles over the XCDs).
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 tm = *reinterpret_cast<const i32x4*>(a.tile_map + 4 * (int64_t)blockIdx.x);
  if (tm.x < 0) return;
  // Uniform values (readfirstlane) keep the K/V bases in SGPRs.
  const int64_t blk = __builtin_amdgcn_readfirstlane(tm.x);  // the block among all query heads' blocks
  const int64_t si = __builtin_amdgcn_readfirstlane(tm.w);
  const SeqAt sa = seq_at_u(a.sq, si, a.block_size);
  const int64_t rb = blk - a.heads * sa.blk0;
  const int64_t hq = rb / sa.nb, j = rb % sa.nb;
  const int64_t e0 = __builtin_amdgcn_readfirstlane(tm.y), e1 = __builtin_amdgcn_readfirstlane(tm.z);
  const int64_t e = e0 + 32 * w + col;
  const bool valid = e < e1;
  const bool wave_on = e0 + 32 * w < e1;
  const int slots = a.k_eff - 1;
  int ev = 0;

  E eng;
  eng.init();
  const T* q = reinterpret_cast<const T*>(a.q);
  // Query rows: read after the first K/V loads are queued. A list entry is
  // the query's global row * slots + slot, which also numbers its partial.
  auto load_q = [&]() {
    ev = a.qlist[valid ? e : e0];
    if (wave_on) eng.load_q(q + (int64_t)(ev / slots) * D, h);
  };
  // Keys and values of the query head's key/value head (grouped-query attention).
  const int64_t kv_heads = a.heads / a.group, kvh = hq / a.group;
  const int64_t kvrow = sa.tok0 * kv_heads + kvh * sa.len + j * a.block_size;
  const T* kp = reinterpret_cast<const T*>(a.k) + kvrow * D;
  const T* vp = reinterpret_cast<const T*>(a.v) + kvrow * D;
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  // The sequence's last block may be short, down to one token; its last
  // subtile then holds fewer than 64 keys.
  const int rows = (int)min<int64_t>(a.block_size, sa.len - j * a.block_size);
  const int nsub = (rows + kSub - 1) / kSub;
  const int last_rows = rows - kSub * (nsub - 1);
  if constexpr (E::kDMA) {
    stream_k_ahead<E, NT>(eng, bufA, bufB, kp, vp, nsub, last_rows, tid, lane, wave_on, sl2, load_q);
  } else {
    stream_subtiles<E, NT>(bufA, bufB, kp, vp, nsub, last_rows, D, tid, load_q, [&](const char* buf, int sub) {
      if (!wave_on) return;
      if (sub == nsub - 1 && last_rows < kSub) eng.template step<true>(buf, lane, 0, last_rows - 1, sl2);
      else eng.template step<false>(buf, lane, 0, 0, sl2);
    });
  }
  if (!wave_on) return;
  const float lt = pair_sum(eng.l);
  if (valid) {
    const int64_t rec = ev;
    T* dst = reinterpret_cast<T*>(a.part_o) + rec * D + h * (D / 2);
    const float inv = 1.f / lt;
#pragma unroll
    for (int dt = 0; dt < E::DT; ++dt) E::put16(dst + 16 * dt, eng.o[dt], inv);
    if (h == 0) a.part_lse[rec] = eng.m + fast_log2(lt);
  }
}

// --------------------------------------------- own block + merge (and dense)
template <typename T, int D, int NW, bool DENSE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(attn_waves<T, D>()))) void
diag_attn_kernel(AttnArgs a) {
  using E = typename EngOf<T, D>::type;
  constexpr int NT = 64 * NW, M = 32 * NW;
  MOBA_KERNEL_LDS(E)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  // Work item -> (sequence, query head, tile of M queries); within a
  // sequence heavier tiles (later in it) come first, heads interleaved.
  constexpr int COL = kSeqW128;
  static_assert(M == 128, "tiles of 128 queries");
  const int64_t item = blockIdx.x;
  const int64_t si = seq_find_u(a.sq, COL, a.heads, item, a.block_size);
  const SeqAt sa = seq_at_u(a.sq, si, a.block_size);
  const int64_t ntile = (sa.len + M - 1) / M;
  const int64_t r_item = item - a.heads * seq_prefix_u(a.sq, si, COL, a.block_size);
  const int64_t tile = ntile - 1 - r_item / a.heads;
  const int64_t hq = r_item % a.heads;
  const int len = (int)sa.len;
  const int64_t row0 = sa.tok0 * a.heads + hq * sa.len;  // row of token 0 of this head
  const int q0 = (int)(tile * M);
  const int qw0 = q0 + 32 * w;
  const int t = qw0 + col;
  // Lanes past the sequence's end (its last tile may be partial) compute on
  // its last query and store nothing.
  const int tq = min(t, len - 1);
  const bool wave_on = qw0 < len;
  // This wave's block c and its keys [kbw, kew); the tile's key stream runs
  // from the block of its first query to its last query (causal), else to
  // the end of that query's block (or, dense, of the sequence); never past
  // the sequence. Subtiles of another wave's block are skipped.
  const int bs = (int)a.block_size;
  const int c = min(qw0, len - 1) / bs;
  const int kbw = DENSE ? 0 : c * bs;
  const int kew = DENSE ? len : min(kbw + bs, len);
  const int qlast = min(q0 + M, len) - 1;
  const int kb = DENSE ? 0 : (q0 / bs) * bs;
  const int kend = a.causal ? qlast + 1 : (DENSE ? len : min((qlast / bs + 1) * bs, len));

  E eng;
  eng.init();
  const T* q = reinterpret_cast<const T*>(a.q);
  // Query rows, and for the own block the merge's seed: run once the first
  // K/V loads are queued, so that their loads overlap.
  auto start = [&]() {
    eng.load_q(q + (row0 + tq) * D, h);
    if (DENSE) return;
    // Start the online softmax from the past-block partials: with
    // m = max lse_i and w_i = 2^(lse_i - m), the state (m, sum w_i,
    // sum w_i o_i) is the partials' union, and the own block's keys then
    // continue it, so the merge needs no pass after the loop. l is kept on
    // one lane of the pair, which sums it at the end.
    const int n_elig = a.causal ? c : (int)sa.nb - 1;
    const int n = min(a.k_eff - 1, n_elig);
    const int slots = a.k_eff - 1;
    const int64_t rec0 = (row0 + tq) * (int64_t)slots;
    if constexpr (sizeof(T) == 2) {
      if (n > 0 && n <= 2) {
        // One or two past blocks (top_k <= 3): every load of both slots is
        // requested before any is used, so the merge waits one memory
        // round trip, not one per load; the arithmetic and its order are
        // those of the general loop below.
        const bf16* po = reinterpret_cast<const bf16*>(a.part_o);
        const bf16* src0 = po + rec0 * D + h * (D / 2);
        const float l0 = a.part_lse[rec0];
        const float l1 = n > 1 ? a.part_lse[rec0 + 1] : kNegInf;
        bf16x8 x0[2 * E::DT], x1[2 * E::DT];
#pragma unroll
        for (int i = 0; i < 2 * E::DT; ++i) x0[i] = *reinterpret_cast<const bf16x8*>(src0 + 8 * i);
        if (n > 1) {
#pragma unroll
          for (int i = 0; i < 2 * E::DT; ++i) x1[i] = *reinterpret_cast<const bf16x8*>(src0 + D + 8 * i);
        }
        const float mx = fmaxf(fmaxf(kNegInf, l0), l1);
        const float w0 = fast_exp2(l0 - mx);
        float wsum = 0.f;
        wsum += w0;
#pragma unroll
        for (int dt = 0; dt < E::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) eng.o[dt][r] = __builtin_fmaf(w0, (float)x0[2 * dt + r / 8][r % 8], eng.o[dt][r]);
        if (n > 1) {
          const float w1 = fast_exp2(l1 - mx);
          wsum += w1;
#pragma unroll
          for (int dt = 0; dt < E::DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              eng.o[dt][r] = __builtin_fmaf(w1, (float)x1[2 * dt + r / 8][r % 8], eng.o[dt][r]);
        }
        eng.m = mx;
        eng.l = h == 0 ? wsum : 0.f;
        return;
      }
    }
    float mx = kNegInf;
    for (int s = 0; s < n; ++s) mx = fmaxf(mx, a.part_lse[rec0 + s]);
    if (n > 0) {
      const T* po = reinterpret_cast<const T*>(a.part_o);
      float wsum = 0.f;
      for (int s = 0; s < n; ++s) {
        const float ws = fast_exp2(a.part_lse[rec0 + s] - mx);
        wsum += ws;
        const T* src = po + (rec0 + s) * D + h * (D / 2);
#pragma unroll
        for (int dt = 0; dt < E::DT; ++dt) {
          float x[16];
          E::get16(src + 16 * dt, x);
#pragma unroll
          for (int r = 0; r < 16; ++r) eng.o[dt][r] = __builtin_fmaf(ws, x[r], eng.o[dt][r]);
        }
      }
      eng.m = mx;
      eng.l = h == 0 ? wsum : 0.f;
    }
  };
  const int64_t kvh = hq / a.group;  // the query head's key/value head
  const int64_t kvrow = sa.tok0 * (a.heads / a.group) + kvh * sa.len + kb;
  const T* kp = reinterpret_cast<const T*>(a.k) + kvrow * D;
  const T* vp = reinterpret_cast<const T*>(a.v) + kvrow * D;
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int nsub = (kend - kb + kSub - 1) / kSub;
  const int last_rows = (kend - kb) - kSub * (nsub - 1);  // keys of the last subtile (1..64)
  // block_size and kb are multiples of 64, so a subtile lies wholly inside
  // or outside the wave's block. Causal: a subtile ending at or before the
  // wave's first query needs no mask (its keys come before every query of
  // the wave and before the sequence's end), one starting after its last
  // query is skipped, the rest are masked at the lane's query. Otherwise
  // only a partial last subtile of the block is masked, at kew - 1.
  const int lim = a.causal ? t : kew - 1;  // the last key a lane may attend
  stream_subtiles<E, NT>(bufA, bufB, kp, vp, nsub, last_rows, D, tid, start, [&](const char* buf, int sub) {
    if (!wave_on) return;
    const int key0 = kb + sub * kSub;
    if (key0 < kbw || key0 >= kew || (a.causal && key0 > qw0 + 31)) return;
    if (key0 + kSub <= (a.causal ? qw0 : kew)) eng.template step<false>(buf, lane, 0, 0, sl2);
    else eng.template step<true>(buf, lane, key0, lim, sl2);
  });
  if (!wave_on) return;

  // Dense, or own block continuing the partials' state: normalise once.
  const float lt = pair_sum(eng.l);
  const float inv = 1.f / lt;
  // The natural-log log-sum-exp of the query's scaled logits over every key
  // it attended (m and l are in the log2 domain), for a backward pass.
  if (t >= len) return;
  if (a.lse_out && h == 0) a.lse_out[row0 + t] = (eng.m + fast_log2(lt)) * 0.69314718f;
#pragma unroll
  for (int dt = 0; dt < E::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) eng.o[dt][r] *= inv;
  T* orow = reinterpret_cast<T*>(a.o) + (row0 + t) * D;
#pragma unroll
  for (int dt = 0; dt < E::DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      E::put4(orow + 32 * dt + 8 * rg + 4 * h, eng.o[dt][4 * rg], eng.o[dt][4 * rg + 1], eng.o[dt][4 * rg + 2],
              eng.o[dt][4 * rg + 3]);
}

namespace {
template <typename K>
hipError_t prep_lds(K kernel, int bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <typename T, int D>
hipError_t gather_t(const AttnArgs& a, hipStream_t s) {
  using E = typename EngOf<T, D>::type;
  constexpr int NW = 4;
  auto kern = gather_attn_kernel<T, D, NW>;
  constexpr int lds = dyn_lds_bytes<E>();
  hipError_t e = prep_lds(kern, lds);
  if (e != hipSuccess) return e;
  const int64_t grid = a.gather_grid;
  KernelTimer timer(s, "gather_attn");
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NW), lds, s, a);
  return hipGetLastError();
}

template <typename T, int D, bool DENSE>
hipError_t diag_t(const AttnArgs& a, hipStream_t s) {
  using E = typename EngOf<T, D>::type;
  // 128-query tiles; a.diag_wgs counts them over all sequences and heads.
  const char* name = DENSE ? "dense_attn" : "diag_merge";
  constexpr int lds = dyn_lds_bytes<E>();
  auto kern = diag_attn_kernel<T, D, 4, DENSE>;
  hipError_t e = prep_lds(kern, lds);
  if (e != hipSuccess) return e;
  KernelTimer timer(s, name);
  hipLaunchKernelGGL(kern, dim3((unsigned)a.diag_wgs), dim3(256), lds, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gather(const AttnArgs& a, hipStream_t s) {
  if (a.bf16_in) return a.head_dim == 128 ? gather_t<bf16, 128>(a, s) : gather_t<bf16, 64>(a, s);
  return a.head_dim == 128 ? gather_t<float, 128>(a, s) : gather_t<float, 64>(a, s);
}
hipError_t launch_diag_merge(const AttnArgs& a, hipStream_t s) {
  if (a.bf16_in) return a.head_dim == 128 ? diag_t<bf16, 128, false>(a, s) : diag_t<bf16, 64, false>(a, s);
  return a.head_dim == 128 ? diag_t<float, 128, false>(a, s) : diag_t<float, 64, false>(a, s);
}
hipError_t launch_dense(const AttnArgs& a, hipStream_t s) {
  if (a.bf16_in) return a.head_dim == 128 ? diag_t<bf16, 128, true>(a, s) : diag_t<bf16, 64, true>(a, s);
  return a.head_dim == 128 ? diag_t<float, 128, true>(a, s) : diag_t<float, 64, true>(a, s);
}


}  // namespace moba
