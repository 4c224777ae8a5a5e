// MoBA backward kernels (bf16 inputs) on the attention engine of
// engine.h; the launch sequence is in api.cpp (moba_backward).
#include "engine.h"

namespace moba {

// ================================================================ backward
// MoBA backward for bf16 inputs, the block choice of the forward held fixed
// (a top-k over block scores has no gradient off ties, and the gate's
// scores do not weight the output): per query, the gradient of one softmax
// attention over its attended keys. With l = q.k / sqrt(D), p = exp(l - lse),
// delta = do . o:  dv_u += p_u do,  ds_u = p_u (do . v_u - delta),
// dq += ds_u k_u / sqrt(D),  dk_u += ds_u q / sqrt(D).
//
// Kernels:
//  bwd_prep    — delta and the log-sum-exp in the log2 domain per query;
//  list_meta   — per list position its query row, log-sum-exp and delta,
//                contiguous (one independent load per row for dK/dV);
//  dq_past     — block-major like gather_attn (the forward's lists and
//                tiles): per 64-key subtile S^T = K Q^T and dP^T = V dO^T on
//                the forward's score path, then dQ^T += K^T dS^T on its P.V
//                path (the same K copy read through the LDS transpose
//                load); subtiles double-buffered; one partial per
//                (query, slot), in bf16 like the forward's output partials;
//  dq_own      — the own block, 128 queries per workgroup (each wave on
//                its own block's keys), causal mask, double-buffered; it
//                then adds the slots' partials in slot order and writes dq
//                (no atomics);
//  dk (x2)     — key-major: a workgroup holds 128 (or 64) keys of one block
//                (32 per wave, as the B operand the way the forward holds
//                queries) and streams 64-row subtiles of the queries that
//                attend them: the block's own queries, then its listed
//                queries (gathered rows), for every query head of the
//                key/value head; blocks in order, heaviest first. One pass
//                accumulates dV^T += dO^T P, the other dK^T += Q^T dS, both
//                on the P.V path; one pass for both would not fit the
//                register file.
namespace {

// C[row][lane column] for 64 LDS rows (K-swizzled layout) against the B
// fragments b (32 columns, one per lane column): the forward's score step.
template <int D>
__device__ __forceinline__ void mm_rows(const char* buf, int lane, const bf16x8 (&b)[D / 16], f32x16 (&c)[2]) {
  using E = EngBF16<D>;
  const int h = lane >> 5, col = lane & 31, sw = E::swz(col);
  const char* r0 = buf + col * E::ROWB;
  const char* r1 = r0 + 32 * E::ROWB;
  c[0] = f32x16{};
  c[1] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(r0 + 16 * ((2 * kk + h) ^ sw));
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(r1 + 16 * ((2 * kk + h) ^ sw));
    c[0] = mfma_bf16(a0, b[kk], c[0]);
    c[1] = mfma_bf16(a1, b[kk], c[1]);
  }
}

// acc^T[d][lane column] += sum over the 64 rows of T[row][d] x[row][column],
// T in LDS read transposed, V-swizzled (VSW; conflict-free) or K-swizzled
// (two-way bank conflicts on these reads, but the same copy serves mm_rows),
// x in the C layout of mm_rows (rounded to bf16): the forward's P.V step.
template <int D, bool VSW = true, bool FENCE = true>
__device__ __forceinline__ void mm_trans(const char* buf, int lane, const f32x16 (&x)[2], f32x16 (&acc)[D / 32]) {
  using E = EngBF16<D>;
  constexpr int DT = D / 32, NP = 4 * DT, VA = 2;  // MFMAs, fragments read ahead
  const int h = lane >> 5, j = lane & 15, half = (lane >> 4) & 1;
  bf16x8 pb[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) pb[nt][r >> 3][r & 7] = to_bf16(x[nt][r]);
  // MFMA c: row chunk c / DT (16 rows), d-tile c % DT. With FENCE the
  // fragments are read VA MFMAs ahead and a scheduling fence after each
  // MFMA keeps the reads from all being hoisted to the front (which would
  // hold every fragment in registers at once); without it the compiler
  // orders them (the dK pass, at the register limit, spills less so).
  auto frag = [&](int c) {
    const int i = c / DT, dt = c % DT, nt = i >> 1, g = i & 1;
    const int d = 32 * dt + 16 * half + 4 * (j & 3);
    const int r0 = 32 * nt + 16 * g + 4 * h + (j >> 2), r1 = r0 + 8;
    const int s0 = VSW ? E::swzv(r0) : E::swz(r0), s1 = VSW ? E::swzv(r1) : E::swz(r1);
    const char* a0 = buf + r0 * E::ROWB + 16 * ((d >> 3) ^ s0) + 2 * (d & 7);
    const char* a1 = buf + r1 * E::ROWB + 16 * ((d >> 3) ^ s1) + 2 * (d & 7);
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a1));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  if constexpr (FENCE) {
    bf16x8 vq[NP];
#pragma unroll
    for (int c = 0; c < VA; ++c) vq[c] = frag(c);
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      if (c + VA < NP) vq[c + VA] = frag(c + VA);
      const int i = c / DT;
      acc[c % DT] = mfma_bf16(vq[c], pb[i >> 1][i & 1], acc[c % DT]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      const int i = c / DT;
      acc[c % DT] = mfma_bf16(frag(c), pb[i >> 1][i & 1], acc[c % DT]);
    }
  }
}

// A row's D/16 B fragments for this lane half (like EngBF16::load_q).
template <int D>
__device__ __forceinline__ void load_frags(bf16x8 (&f)[D / 16], const bf16* row, int h) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = *reinterpret_cast<const bf16x8*>(row + 16 * kk + 8 * h);
}

// acc (C layout of mm_trans: lane column = row of dst, element r = coordinate
// 32 dt + crow(r, h)) times scale, to a bf16 row of dst.
template <int D>
__device__ __forceinline__ void store_row_bf16(bf16* dst, const f32x16 (&acc)[D / 32], int h, float scale) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      EngBF16<D>::put4(dst + 32 * dt + 8 * rg + 4 * h, acc[dt][4 * rg] * scale, acc[dt][4 * rg + 1] * scale,
                       acc[dt][4 * rg + 2] * scale, acc[dt][4 * rg + 3] * scale);
}

// 64 rows of src (rows[i] = row index, from LDS) into buf, K-swizzled
// (V = false) or V-swizzled (V = true), by direct HBM -> LDS loads.
template <int D, int NT, bool V>
__device__ __forceinline__ void load_rows(const bf16* src, const int* rows, char* buf, int tid) {
  using E = EngBF16<D>;
  constexpr int NW = NT / 64, INSTS = E::SLOTS / 64;
  static_assert(INSTS % NW == 0, "subtile slots must split evenly over the waves");
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const unsigned base = __builtin_amdgcn_readfirstlane(lds_addr(buf));
#pragma unroll
  for (int ii = 0; ii < INSTS / NW; ++ii) {
    const int i = ii * NW + w;
    const int sl = i * 64 + lane;
    const int row = sl / E::CPR;
    const int x = (sl % E::CPR) ^ (V ? E::swzv(row) : E::swz(row));
    lds_dma16(src + (int64_t)rows[row] * D + 8 * x, base + i * 1024);
  }
}

__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const int tid = threadIdx.x, sub = tid & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const int64_t n = a.bh * a.seq_len;
  const int D = a.head_dim;
  float sum = 0.f;
  if (row < n) {
    // 16 lanes per row, one 16-byte (D = 128) or 8-byte (D = 64) load each.
    const bf16* o = reinterpret_cast<const bf16*>(a.o) + row * D;
    const bf16* g = reinterpret_cast<const bf16*>(a.dout) + row * D;
    if (D == 128) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(o + 8 * sub);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(g + 8 * sub);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum = __builtin_fmaf((float)x[e], (float)y[e], sum);
    } else {
      const bf16x4 x = *reinterpret_cast<const bf16x4*>(o + 4 * sub);
      const bf16x4 y = *reinterpret_cast<const bf16x4*>(g + 4 * sub);
#pragma unroll
      for (int e = 0; e < 4; ++e) sum = __builtin_fmaf((float)x[e], (float)y[e], sum);
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) sum += __shfl_xor(sum, m);
  if (row < n && sub == 0) {
    a.delta[row] = sum;
    a.lse2[row] = a.lse[row] * kLog2e;
  }
}

// One key subtile of a dq workgroup: p and ds from the scores, dq^T += K^T ds.
template <int D, bool MASK>
__device__ __forceinline__ void dq_step(const char* bk, const char* bv, int lane,
                                        const bf16x8 (&qf)[D / 16], const bf16x8 (&gf)[D / 16], float lse2,
                                        float delta, float sl2, int key0, int t, f32x16 (&acc)[D / 32]) {
  const int h = lane >> 5;
  f32x16 s[2], dp[2];
  mm_rows<D>(bk, lane, qf, s);
  mm_rows<D>(bv, lane, gf, dp);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(__builtin_fmaf(s[nt][r], sl2, -lse2));
      if (MASK && key0 + 32 * nt + crow(r, h) > t) p = 0.f;
      s[nt][r] = p * (dp[nt][r] - delta);
    }
  mm_trans<D, false>(bk, lane, s, acc);
}

// Past blocks: one gather tile (a block and up to 128 listed queries).
// TAIL: the sequence length is not a multiple of 64, so a block's last
// subtile may be partial.
template <int D, bool TAIL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void dq_past_kernel(BwdArgs a) {
  using E = EngBF16<D>;
  constexpr int NT = 256, KC = D / 16, DT = D / 32;
  __shared__ __align__(16) char bk0[E::TB], bv0[E::TB], bk1[E::TB], bv1[E::TB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 tm = *reinterpret_cast<const i32x4*>(a.tile_map + 4 * (int64_t)blockIdx.x);
  if (tm.x < 0) return;
  const int64_t blk = __builtin_amdgcn_readfirstlane(tm.x);
  const int64_t bh = blk / a.n_blocks, j = blk % a.n_blocks;
  const int64_t e0 = __builtin_amdgcn_readfirstlane(tm.y), e1 = __builtin_amdgcn_readfirstlane(tm.z);
  const int64_t e = e0 + 32 * w + col;
  const bool valid = e < e1, wave_on = e0 + 32 * w < e1;
  const int slots = a.k_eff - 1;
  const int ev = a.qlist[valid ? e : e0];  // the query's global row * slots + slot
  const int64_t row = ev / slots;
  bf16x8 qf[KC], gf[KC];
  load_frags<D>(qf, reinterpret_cast<const bf16*>(a.q) + row * D, h);
  load_frags<D>(gf, reinterpret_cast<const bf16*>(a.dout) + row * D, h);
  const float lse2 = a.lse2[row], delta = a.delta[row];
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int64_t kvh = bh / a.group;
  const bf16* kp = reinterpret_cast<const bf16*>(a.k) + (kvh * a.seq_len + j * a.block_size) * D;
  const bf16* vp = reinterpret_cast<const bf16*>(a.v) + (kvh * a.seq_len + j * a.block_size) * D;
  // The block's keys (the sequence's last block may be short, its last
  // subtile partial: rows past its end are loaded as copies and masked).
  const int nkeys = (int)min<int64_t>(a.block_size, a.seq_len - j * a.block_size);
  const int nsub = (nkeys + kSub - 1) / kSub;
  const int last_rows = nkeys - kSub * (nsub - 1);
  auto rows_of = [&](int sub) { return TAIL && sub == nsub - 1 ? last_rows : kSub; };
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  // Double-buffered: the loads of subtile sub + 1 run under the compute of
  // sub (buffer sub & 1); each step ends waiting for them, then the barrier.
  E::template begin_one<NT, false>(kp, bk0, tid, rows_of(0));
  E::template begin_one<NT, false>(vp, bv0, tid, rows_of(0));
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), also for the query rows
  lds_dma_wait();
  __syncthreads();
  for (int sub = 0; sub < nsub; ++sub) {
    const bool odd = sub & 1;
    if (sub + 1 < nsub) {
      E::template begin_one<NT, false>(kp + (int64_t)(sub + 1) * kSub * D, odd ? bk0 : bk1, tid, rows_of(sub + 1));
      E::template begin_one<NT, false>(vp + (int64_t)(sub + 1) * kSub * D, odd ? bv0 : bv1, tid, rows_of(sub + 1));
    }
    // With TAIL one masked step serves every subtile (keys past the
    // subtile's rows get no weight; a full subtile masks nothing): a second,
    // unmasked copy of the step would push the kernel past the register
    // file.
    if (wave_on) {
      if constexpr (TAIL)
        dq_step<D, true>(odd ? bk1 : bk0, odd ? bv1 : bv0, lane, qf, gf, lse2, delta, sl2, 0, rows_of(sub) - 1, acc);
      else
        dq_step<D, false>(odd ? bk1 : bk0, odd ? bv1 : bv0, lane, qf, gf, lse2, delta, sl2, 0, 0, acc);
    }
    lds_dma_wait();
    __syncthreads();
  }
  if (valid) store_row_bf16<D>(a.dq_part + (int64_t)ev * D, acc, h, 1.f / __builtin_sqrtf((float)D));
}

// The own block: 128 consecutive queries of one head, 32 per wave. A
// wave's queries share one block (block_size is a multiple of 64); the
// workgroup's may span blocks, and each wave takes only its own block's
// subtiles of the workgroup's key stream. The sequence's last tile may be
// partial: waves past its end compute nothing, lanes past it compute on
// its last query and store nothing, and its last key subtile may be
// partial (rows past the end are loaded as copies and masked; TAIL: the
// length is not a multiple of 64).
template <int D, bool TAIL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void dq_own_kernel(BwdArgs a) {
  using E = EngBF16<D>;
  constexpr int NT = 256, KC = D / 16, DT = D / 32, M = 128;
  // Double-buffered (64 KB): registers already limit a compute unit to two
  // of these workgroups (four waves each), which the LDS still holds.
  __shared__ __align__(16) char bk0[E::TB], bv0[E::TB], bk1[E::TB], bv1[E::TB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  const int64_t ntile = (a.seq_len + M - 1) / M;
  const int64_t bh = blockIdx.x / ntile;
  const int q0 = (int)((blockIdx.x % ntile) * M);
  const int len = (int)a.seq_len, bs = (int)a.block_size;
  const int qw0 = q0 + 32 * w;
  const bool wave_on = qw0 < len;
  // This wave's block c and its keys [kbw, kew); the stream runs from the
  // block of the tile's first query to its last query (causal), else to
  // the end of that query's block.
  const int c = min(qw0, len - 1) / bs;
  const int kbw = c * bs, kew = min(kbw + bs, len);
  const int qlast = min(q0 + M, len) - 1;
  const int kb = (q0 / bs) * bs;
  const int kend = a.causal ? qlast + 1 : min((qlast / bs + 1) * bs, len);
  const bool lane_on = TAIL ? qw0 + col < len : wave_on;
  const int t = lane_on ? qw0 + col : len - 1;
  const int64_t row = bh * a.seq_len + t;
  bf16x8 qf[KC], gf[KC];
  load_frags<D>(qf, reinterpret_cast<const bf16*>(a.q) + row * D, h);
  load_frags<D>(gf, reinterpret_cast<const bf16*>(a.dout) + row * D, h);
  const float lse2 = a.lse2[row], delta = a.delta[row];
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int64_t kvh = bh / a.group;
  const bf16* kp = reinterpret_cast<const bf16*>(a.k) + (kvh * a.seq_len + kb) * D;
  const bf16* vp = reinterpret_cast<const bf16*>(a.v) + (kvh * a.seq_len + kb) * D;
  const int nsub = (kend - kb + kSub - 1) / kSub;
  const int last_rows = (kend - kb) - kSub * (nsub - 1);
  auto rows_of = [&](int sub) { return TAIL && sub == nsub - 1 ? last_rows : kSub; };
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  E::template begin_one<NT, false>(kp, bk0, tid, rows_of(0));
  E::template begin_one<NT, false>(vp, bv0, tid, rows_of(0));
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), also for the query rows
  lds_dma_wait();
  __syncthreads();
  for (int sub = 0; sub < nsub; ++sub) {
    // Subtile sub is in buffer sub & 1; sub + 1 loads into the other one
    // (last read in step sub - 1, before its barrier).
    const bool odd = sub & 1;
    if (sub + 1 < nsub) {
      E::template begin_one<NT, false>(kp + (int64_t)(sub + 1) * kSub * D, odd ? bk0 : bk1, tid, rows_of(sub + 1));
      E::template begin_one<NT, false>(vp + (int64_t)(sub + 1) * kSub * D, odd ? bv0 : bv1, tid, rows_of(sub + 1));
    }
    const char* bk = odd ? bk1 : bk0;
    const char* bv = odd ? bv1 : bv0;
    const int key0 = kb + sub * kSub;
    // Causal: masked at the lane's query on the diagonal (which also masks
    // keys past the sequence's end), skipped past the wave's last query.
    // Otherwise only a partial last subtile of the block is masked, at
    // kew - 1. With TAIL one masked step serves every subtile (a second,
    // unmasked copy of the step would push the kernel past the register
    // file).
    if constexpr (TAIL) {
      if (wave_on && key0 >= kbw && key0 < kew && !(a.causal && key0 > qw0 + 31)) {
        const bool need = key0 + kSub > (a.causal ? qw0 : kew);
        const int lim = need ? (a.causal ? t : kew - 1) : key0 + kSub - 1;
        dq_step<D, true>(bk, bv, lane, qf, gf, lse2, delta, sl2, key0, lim, acc);
      }
    } else if (wave_on && key0 >= kbw && key0 < kew) {
      if (a.causal && key0 + kSub > qw0) {
        if (key0 <= qw0 + 31) dq_step<D, true>(bk, bv, lane, qf, gf, lse2, delta, sl2, key0, t, acc);
      } else {
        dq_step<D, false>(bk, bv, lane, qf, gf, lse2, delta, sl2, 0, 0, acc);
      }
    }
    lds_dma_wait();
    __syncthreads();
  }
  if (!lane_on) return;
  // dq = own-block part + the past slots' bf16 partials (written by
  // dq_past, an earlier launch), added in fp32 in slot order and rounded
  // to bf16.
  const float scale = 1.f / __builtin_sqrtf((float)D);
  // The row's past blocks, counted as the list-building kernels count them
  // (the same validity test and cap), so exactly the partials dq_past wrote.
  const int slots = a.k_eff - 1;
  const int cap = past_cap(c, a.n_blocks, a.causal, a.k_eff);
  int n = 0;
  {
    const int32_t* ir = a.block_idx + row * a.top_k;
    for (int i = 0; i < a.top_k && n < cap; ++i) {
      const int j = ir[i];
      if (j < 0) break;
      n += routed_past_block(j, c, a.n_blocks, a.causal) ? 1 : 0;
    }
  }
  bf16* dst = reinterpret_cast<bf16*>(a.dq) + row * D;
  const bf16* p0 = a.dq_part + (row * slots) * D;
  auto ld4 = [](const bf16* p) {
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
  };
  if (n <= 2) {
    // One or two past blocks (top_k <= 3): every partial is requested
    // before any is added (one memory round trip); slot order kept (the
    // own part's scaling may fuse with the first addition).
    f32x4 y0[DT * 4], y1[DT * 4];
#pragma unroll
    for (int i = 0; i < DT * 4; ++i) {
      const int d = 32 * (i / 4) + 8 * (i % 4) + 4 * h;
      if (n > 0) y0[i] = ld4(p0 + d);
      if (n > 1) y1[i] = ld4(p0 + D + d);
    }
#pragma unroll
    for (int i = 0; i < DT * 4; ++i) {
      const int dt = i / 4, rg = i % 4, d = 32 * dt + 8 * rg + 4 * h;
      f32x4 x = f32x4{acc[dt][4 * rg] * scale, acc[dt][4 * rg + 1] * scale, acc[dt][4 * rg + 2] * scale,
                      acc[dt][4 * rg + 3] * scale};
      if (n > 0) x += y0[i];
      if (n > 1) x += y1[i];
      E::put4(dst + d, x[0], x[1], x[2], x[3]);
    }
    return;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = 32 * dt + 8 * rg + 4 * h;
      f32x4 x = f32x4{acc[dt][4 * rg] * scale, acc[dt][4 * rg + 1] * scale, acc[dt][4 * rg + 2] * scale,
                      acc[dt][4 * rg + 3] * scale};
      for (int sl = 0; sl < n; ++sl) x += ld4(p0 + sl * D + d);
      E::put4(dst + d, x[0], x[1], x[2], x[3]);
    }
}

// Per list position (the forward's lists, rebuilt in a fixed order): the
// query row, its log-sum-exp and its delta, stored contiguously so that the
// dK/dV passes read a subtile's metadata with one independent load each.
__global__ __launch_bounds__(256) void list_meta_kernel(BwdArgs a) {
  const int64_t lst = blockIdx.x;  // bh * n_blocks + j
  const int64_t bh = lst / a.n_blocks;
  const int slots = a.k_eff - 1;
  const int o0 = a.offset[lst], o1 = a.offset[lst + 1];
  for (int pos = o0 + (int)threadIdx.x; pos < o1; pos += 256) {
    const int64_t row = a.qlist[pos] / slots;  // global query row (bh * seq_len + t)
    a.lt[pos] = (int32_t)(row - bh * a.seq_len);
    a.ll[pos] = a.lse2[row];
    a.ld[pos] = a.delta[row];
  }
}

// dV (PASS = 0) or dK (PASS = 1) for 32 * NW keys of one block of one
// key/value head, single-buffered: each 64-row query subtile is staged
// (row numbers, log-sum-exps and deltas, for listed rows from
// list_meta_kernel's contiguous arrays, then the rows of Q and dO) and
// then computed; dV^T += dO^T P reads dO transposed from a V-swizzled copy,
// dK^T += Q^T dS reads Q transposed from its one K-swizzled copy. The dV
// pass (168 registers) runs at three waves per SIMD, three workgroups of
// 32 KB of LDS per compute unit, which hides the row gathers' latency
// better than two waves of a two-buffer pipeline; the dK pass holds K and V
// fragments besides its accumulators and runs at two.
template <int D, int PASS, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(PASS == 0 ? 3 : 2))) void
dk_kernel(BwdArgs a) {
  using E = EngBF16<D>;
  constexpr int NT = 64 * NW, KC = D / 16, DT = D / 32, KEYS = 32 * NW;
  __shared__ __align__(16) char bq[E::TB], bx[E::TB];
  __shared__ int rows[64];
  __shared__ float lse2s[64], deltas[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  // Blocks in order, all heads of a block together: early blocks are in
  // the most lists (causal routing), so the longest workgroups start first.
  const int64_t nchunk = a.block_size / KEYS;
  const int64_t nkv = a.bh / a.group;
  const int64_t kc = blockIdx.x % nchunk;
  const int64_t kvh = (blockIdx.x / nchunk) % nkv;
  const int64_t j = blockIdx.x / (nchunk * nkv);
  const int64_t k0 = j * a.block_size + kc * KEYS;
  if (k0 >= a.seq_len) return;  // past the end of a short last block
  // This lane's key; lanes past the sequence's end compute on its last
  // key and store nothing.
  const int u = (int)k0 + 32 * w + col;
  const int uc = min(u, (int)a.seq_len - 1);
  const bf16* krow = reinterpret_cast<const bf16*>(a.k) + (kvh * a.seq_len + uc) * D;
  const bf16* vrow = reinterpret_cast<const bf16*>(a.v) + (kvh * a.seq_len + uc) * D;
  bf16x8 kf[KC], vf[PASS == 1 ? KC : 1];
  load_frags<D>(kf, krow, h);
  if constexpr (PASS == 1) load_frags<D>(vf, vrow, h);
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int slots = a.k_eff - 1;
  const int64_t jend = min<int64_t>((j + 1) * a.block_size, a.seq_len);
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  // One 64-row subtile of query head bh, n valid rows from `first`: own
  // rows are consecutive queries (masked against the keys when causal),
  // listed rows are list positions.
  auto subtile = [&](int64_t bh, int n, bool own, int64_t first) {
    const bool mask = own && a.causal;
    if (tid < 64) {
      const bool ok = tid < n;
      const int64_t i = first + (ok ? tid : 0);  // a padding row repeats a valid one
      int t;
      float l, dl;
      if (own) {
        t = (int)i;
        l = a.lse2[bh * a.seq_len + i];
        dl = a.delta[bh * a.seq_len + i];
      } else {  // list position: one independent load each
        t = a.lt[i];
        l = a.ll[i];
        dl = a.ld[i];
      }
      rows[tid] = t;
      lse2s[tid] = ok ? l : __builtin_inff();
      deltas[tid] = ok ? dl : 0.f;
    }
    __syncthreads();
    const bf16* qb = reinterpret_cast<const bf16*>(a.q) + bh * a.seq_len * D;
    const bf16* gb = reinterpret_cast<const bf16*>(a.dout) + bh * a.seq_len * D;
    load_rows<D, NT, false>(qb, rows, bq, tid);
    if constexpr (PASS == 0) {
      load_rows<D, NT, true>(gb, rows, bx, tid);   // dO^T for dV
    } else {
      load_rows<D, NT, false>(gb, rows, bx, tid);  // dO for dP
    }
    lds_dma_wait();
    __syncthreads();
    f32x16 s[2];
    mm_rows<D>(bq, lane, kf, s);
    f32x16 dp[2];
    if constexpr (PASS == 1) mm_rows<D>(bx, lane, vf, dp);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int r0 = 32 * nt + 8 * rg + 4 * h;  // rows of elements 4 rg .. 4 rg + 3
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + r0);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(deltas + r0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          float p = fast_exp2(__builtin_fmaf(s[nt][r], sl2, -l4[e]));
          if (mask && u > rows[r0 + e]) p = 0.f;
          if constexpr (PASS == 0) s[nt][r] = p;
          else s[nt][r] = p * (dp[nt][r] - d4[e]);
        }
      }
    if constexpr (PASS == 0) mm_trans<D>(bx, lane, s, acc);
    else mm_trans<D, false, false>(bq, lane, s, acc);
    __syncthreads();
  };
  for (int g = 0; g < a.group; ++g) {
    const int64_t bh = kvh * a.group + g;
    // The block's own queries: those at or after the keys (causal), or all.
    const int64_t qs = a.causal ? k0 : j * a.block_size;
    for (int64_t t0 = qs; t0 < jend; t0 += 64) {
      const int n = (int)min<int64_t>(64, jend - t0);
      subtile(bh, n, true, t0);
    }
    // Its listed queries (past-block routing of later, or other, queries).
    if (slots > 0) {
      const int64_t o0 = a.offset[bh * a.n_blocks + j];
      const int cnt = a.offset[bh * a.n_blocks + j + 1] - o0;
      for (int i0 = 0; i0 < cnt; i0 += 64) subtile(bh, min(64, cnt - i0), false, o0 + i0);
    }
  }
  if (u >= a.seq_len) return;
  bf16* dst = reinterpret_cast<bf16*>(PASS == 0 ? a.dv : a.dk) + (kvh * a.seq_len + u) * D;
  store_row_bf16<D>(dst, acc, h, PASS == 0 ? 1.f : 1.f / __builtin_sqrtf((float)D));
}

template <int D>
hipError_t backward_t(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = a.bh * a.seq_len;
  const bool tail = a.seq_len % kSub != 0;  // partial last query tiles and key subtiles
  {
    KernelTimer t(s, "bwd_prep");
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.k_eff > 1 && a.gather_grid > 0) {
    KernelTimer t(s, "bwd_list_meta");
    hipLaunchKernelGGL(list_meta_kernel, dim3((unsigned)(a.bh * a.n_blocks)), dim3(256), 0, s, a);
  }
  if (a.k_eff > 1 && a.gather_grid > 0) {
    KernelTimer t(s, "bwd_dq_past");
    if (tail) hipLaunchKernelGGL((dq_past_kernel<D, true>), dim3((unsigned)a.gather_grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dq_past_kernel<D, false>), dim3((unsigned)a.gather_grid), dim3(256), 0, s, a);
  }
  {
    KernelTimer t(s, "bwd_dq_own");
    const dim3 grid((unsigned)(a.bh * ((a.seq_len + 127) / 128)));
    if (tail) hipLaunchKernelGGL((dq_own_kernel<D, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dq_own_kernel<D, false>), grid, dim3(256), 0, s, a);
  }
  // 128 keys per workgroup where every block length is a multiple of 128,
  // else 64.
  const int64_t last = a.seq_len - (a.n_blocks - 1) * a.block_size;
  const bool wide = a.block_size % 128 == 0 && last % 128 == 0;
  const int64_t kv_wgs = (a.bh / a.group) * a.n_blocks * (a.block_size / (wide ? 128 : 64));
  // dK before dV: in that order both passes ran faster in a same-box A/B
  // (4.56 against 4.62 ms per backward at headline_32k).
  {
    KernelTimer t(s, "bwd_dk");
    if (wide) hipLaunchKernelGGL((dk_kernel<D, 1, 4>), dim3((unsigned)kv_wgs), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dk_kernel<D, 1, 2>), dim3((unsigned)kv_wgs), dim3(128), 0, s, a);
  }
  {
    KernelTimer t(s, "bwd_dv");
    if (wide) hipLaunchKernelGGL((dk_kernel<D, 0, 4>), dim3((unsigned)kv_wgs), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dk_kernel<D, 0, 2>), dim3((unsigned)kv_wgs), dim3(128), 0, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? backward_t<128>(a, s) : backward_t<64>(a, s);
}

}  // namespace moba
