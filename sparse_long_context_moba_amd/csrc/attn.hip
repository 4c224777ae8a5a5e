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
//  diag_merge   — the own block. A workgroup takes 32*NW consecutive queries
//                 of one block, starts each query's online softmax from its
//                 past partials (the log-sum-exp merge, done first), attends
//                 the block's keys up to the query (causal) and writes o in
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
#include "common.h"
#include "launch.h"

namespace moba {
namespace {

constexpr int kSub = 64;  // keys per LDS subtile
constexpr float kLog2e = 1.4426950408889634f;

// Max / sum of a value over the two lanes (l, l^32) that hold one query.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online-softmax update shared by both engines. s holds raw scores of 64
// keys for this lane's query; on return it holds the weights
// exp2(s*sl2 - m). m is the running reference (log2 domain); it is raised
// only when a row's maximum exceeds it by more than 8, so weights stay
// below 2^8 and the output accumulators are rescaled rarely.
template <bool MASK, int DT>
__device__ __forceinline__ void online_softmax(f32x16 (&s)[2], float& m, float& l, f32x16 (&o)[DT], int h,
                                               int key0, int qpos, float sl2) {
  if (MASK) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + 32 * nt + crow(r, h) > qpos) s[nt][r] = kNegInf;
  }
  float mx = kNegInf;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[nt][r], s[nt][r + 1]));
  mx = pair_max(mx) * sl2;
  if (__builtin_amdgcn_ballot_w64(mx > m + 8.f)) {
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    m = mn;
  }
  const float nm = -m;
  float rs = 0.f;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(__builtin_fmaf(s[nt][r], sl2, nm));
      s[nt][r] = e;
      rs += e;
    }
  l += rs;
}

// ------------------------------------------------------------ bf16 engine
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_base + 16*l, lds_base being wave-uniform.
// Issued from inline assembly so that the compiler does not make unrelated
// LDS reads wait for it; the caller waits explicitly (lds_dma_wait) before
// the barrier that publishes the data.
__device__ __forceinline__ void lds_dma16(const void* src, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base) : "memory");
}
// The same with a wave-uniform base address (SGPR pair) and a 32-bit
// per-lane byte offset, so no per-load 64-bit address arithmetic.
__device__ __forceinline__ void lds_dma16_s(const void* base, unsigned off, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds_base) : "memory");
}
__device__ __forceinline__ void lds_dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ unsigned lds_addr(const char* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

template <int D>
struct EngBF16 {
  using T = bf16;
  static constexpr bool kDMA = true;
  static constexpr int kD = D;
  static constexpr int KC = D / 16, DT = D / 32;
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int ROWB = D * 2;       // bytes per K/V row in LDS
  static constexpr int TB = kSub * ROWB;   // bytes of one K (or V) subtile
  static constexpr int BUF_BYTES = 2 * TB; // K subtile, then V subtile
  static constexpr int SLOTS = kSub * CPR; // 16-byte slots per subtile

  bf16x8 qf[KC];
  f32x16 o[DT];
  float m, l;

  template <int NT>
  struct Stage {};

  // Physical chunk of logical chunk x in row r is x ^ swz(r) for K and
  // x ^ swzv(r) for V. LDS serves 256 bytes (64 banks) per cycle: 16 lanes
  // of a 16-byte read or 32 lanes of an 8-byte read.
  //  - K reads: 16 consecutive rows at one logical chunk. swz is a bijection
  //    of r % 16 (D = 128, a row spans the 64 banks) or of (r / 2) % 8 within
  //    each parity (D = 64, two rows span them).
  //  - V transpose reads: 4 aligned rows x logical chunks x0 .. x0+3 (x0 a
  //    multiple of 4) per 32 lanes. swzv only moves whole 64-byte segments:
  //    bits 2-3 differ across the 4 rows (D = 128), or bit 2 differs between
  //    rows of equal parity (D = 64).
  static __device__ __forceinline__ int swz(int r) {
    return CPR == 16 ? ((2 * (r & 7)) | ((r >> 3) & 1)) : ((2 * (r & 3)) | ((r >> 2) & 1));
  }
  static __device__ __forceinline__ int swzv(int r) {
    return CPR == 16 ? (4 * (r & 3)) : (((r >> 1) & 1) << 2);
  }

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    m = kNegInf;
    l = 0.f;
  }
  __device__ __forceinline__ void load_q(const bf16* qrow, int h) {
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk + 8 * h);
  }

  // Queue the direct HBM -> LDS loads of one K and one V subtile (64 rows
  // each) into buf. Each wave instruction fills 64 consecutive 16-byte slots;
  // the lane picks the source chunk that belongs in its slot.
  template <int NT>
  static __device__ __forceinline__ void begin(Stage<NT>&, const bf16* kp, const bf16* vp, char* buf, int tid) {
    constexpr int NW = NT / 64, INSTS = SLOTS / 64;
    static_assert(INSTS % NW == 0, "subtile slots must split evenly over the waves");
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned base = __builtin_amdgcn_readfirstlane(lds_addr(buf));
#pragma unroll
    for (int ii = 0; ii < INSTS / NW; ++ii) {
      const int i = ii * NW + w;
      const int sl = i * 64 + lane;
      const int row = sl / CPR, x = (sl % CPR) ^ swz(sl / CPR);
      lds_dma16(kp + row * D + 8 * x, base + i * 1024);
      lds_dma16(vp + row * D + 8 * ((sl % CPR) ^ swzv(row)), base + TB + i * 1024);
    }
  }
  // Wait for this wave's queued loads (the caller's barrier covers the rest).
  template <int NT>
  static __device__ __forceinline__ void land(Stage<NT>&, char*, int) {
    lds_dma_wait();
  }
  // Direct loads one wave issues for one K (or V) subtile.
  template <int NT>
  static constexpr int kLoadsPerWave = SLOTS / 64 / (NT / 64);
  // Per-lane source offsets (bytes from the subtile's first row) of this
  // wave's loads of one K (v = false) or V (v = true) subtile.
  template <int NT>
  struct LoadOffsets {
    unsigned k[kLoadsPerWave<NT>], v[kLoadsPerWave<NT>];
  };
  template <int NT>
  static __device__ __forceinline__ void load_offsets(LoadOffsets<NT>& lo, int tid) {
    constexpr int NW = NT / 64;
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int ii = 0; ii < kLoadsPerWave<NT>; ++ii) {
      const int sl = (ii * NW + w) * 64 + lane, row = sl / CPR;
      lo.k[ii] = (unsigned)(row * D + 8 * ((sl % CPR) ^ swz(row))) * 2u;
      lo.v[ii] = (unsigned)(row * D + 8 * ((sl % CPR) ^ swzv(row))) * 2u;
    }
  }
  // The loads of one subtile from a wave-uniform base p.
  template <int NT, bool IS_V>
  static __device__ __forceinline__ void begin_uniform(const bf16* p, const LoadOffsets<NT>& lo, char* buf, int tid) {
    constexpr int NW = NT / 64;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned base = __builtin_amdgcn_readfirstlane(lds_addr(buf));
#pragma unroll
    for (int ii = 0; ii < kLoadsPerWave<NT>; ++ii)
      lds_dma16_s(p, IS_V ? lo.v[ii] : lo.k[ii], base + (ii * NW + w) * 1024);
  }
  // The same loads for K or V alone, into a buffer of TB bytes.
  template <int NT, bool IS_V>
  static __device__ __forceinline__ void begin_one(const bf16* p, char* buf, int tid) {
    constexpr int NW = NT / 64, INSTS = SLOTS / 64;
    static_assert(INSTS % NW == 0, "subtile slots must split evenly over the waves");
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned base = __builtin_amdgcn_readfirstlane(lds_addr(buf));
#pragma unroll
    for (int ii = 0; ii < INSTS / NW; ++ii) {
      const int i = ii * NW + w;
      const int sl = i * 64 + lane;
      const int row = sl / CPR;
      const int x = (sl % CPR) ^ (IS_V ? swzv(row) : swz(row));
      lds_dma16(p + row * D + 8 * x, base + i * 1024);
    }
  }

  // ---- the step in parts, for the pipelined stream (K one subtile ahead
  // of V): scores of a K subtile, their row maximum, the lazy rescale, and
  // the weights and P.V of an earlier subtile.
  __device__ __forceinline__ void qk(const char* kbuf, int lane, f32x16 (&s)[2]) const {
    const int h = lane >> 5, col = lane & 31;
    const int sw = swz(col);
    const char* r0 = kbuf + col * ROWB;
    const char* r1 = r0 + 32 * ROWB;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(r0 + 16 * ((2 * kk + h) ^ sw));
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(r1 + 16 * ((2 * kk + h) ^ sw));
      s[0] = mfma_bf16(a0, qf[kk], s[0]);
      s[1] = mfma_bf16(a1, qf[kk], s[1]);
    }
  }
  // Scaled (log2-domain) maximum of the query's 64 scores.
  static __device__ __forceinline__ float rowmax(const f32x16 (&s)[2], float sl2) {
    float a = kNegInf, b = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      a = fmaxf(a, fmaxf(s[0][r], s[0][r + 1]));
      b = fmaxf(b, fmaxf(s[1][r], s[1][r + 1]));
    }
    return pair_max(fmaxf(a, b)) * sl2;
  }
  // Raise the reference to cover mx (see online_softmax).
  __device__ __forceinline__ void rescale(float mx) {
    if (__builtin_amdgcn_ballot_w64(mx > m + 8.f)) {
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m = mn;
    }
  }
  // Weights exp2(s * sl2 - m) of the scores in s, added to l, and O += P V
  // with V from vbuf (one subtile, TB bytes).
  __device__ __forceinline__ void expo_pv(const f32x16 (&s)[2], const char* vbuf, int lane, float sl2) {
    const int h = lane >> 5;
    const float nm = -m;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8 pb[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(s[nt][r], sl2, nm));
        rs[r & 3] += e;
        pb[nt][r >> 3][r & 7] = to_bf16(e);
      }
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    const int j = lane & 15, half = (lane >> 4) & 1;
    // Key chunks outer, d-tiles inner: consecutive MFMAs accumulate into
    // different tiles.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int nt = i >> 1, g = i & 1;
        const int d = 32 * dt + 16 * half + 4 * (j & 3);
        const int r0 = 32 * nt + 16 * g + 4 * h + (j >> 2), r1 = r0 + 8;
        const char* a0 = vbuf + r0 * ROWB + 16 * ((d >> 3) ^ swzv(r0)) + 2 * (d & 7);
        const char* a1 = vbuf + r1 * ROWB + 16 * ((d >> 3) ^ swzv(r1)) + 2 * (d & 7);
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a1));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = mfma_bf16(vf, pb[nt][g], o[dt]);
      }
  }
  // The steady-state step of the pipelined stream, in issue order (waves
  // issue in order, so the MFMA chains only hide the softmax arithmetic if
  // the two are interleaved in the instruction stream): scores of the next
  // K subtile (kbn -> sn) with the weights of the current scores sc, then
  // O += P V from vbc with the row maximum of sn. Each chunk ends in a
  // scheduling fence; fragments are read a few chunks ahead.
  __device__ __forceinline__ void fused(const char* kbn, f32x16 (&sn)[2], const f32x16 (&sc)[2], const char* vbc,
                                        int lane, float sl2, float& mxn) {
    const int h = lane >> 5, col = lane & 31, sw = swz(col);
    const char* kr0 = kbn + col * ROWB;
    const char* kr1 = kr0 + 32 * ROWB;
    // QK MFMA c: key half c % 2, k-chunk c / 2.
    auto kfrag = [&](int c) {
      return *reinterpret_cast<const bf16x8*>(((c & 1) ? kr1 : kr0) + 16 * ((2 * (c >> 1) + h) ^ sw));
    };
    const int j = lane & 15, half = (lane >> 4) & 1;
    // P.V MFMA c: d-tile c % DT, keys 16 * (c / DT) .. +15 (consecutive
    // MFMAs accumulate into different tiles).
    auto vfrag = [&](int c) {
      const int dt = c % DT, nt = (c / DT) >> 1, g = (c / DT) & 1;
      const int d = 32 * dt + 16 * half + 4 * (j & 3);
      const int r0 = 32 * nt + 16 * g + 4 * h + (j >> 2), r1 = r0 + 8;
      const char* a0 = vbc + r0 * ROWB + 16 * ((d >> 3) ^ swzv(r0)) + 2 * (d & 7);
      const char* a1 = vbc + r1 * ROWB + 16 * ((d >> 3) ^ swzv(r1)) + 2 * (d & 7);
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a1));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int NQ = 2 * KC, NP = 4 * DT, KA = 3, VA = 2;
    static_assert(NQ == 16 || NQ == 8, "32 score pairs over the QK chunks");
    constexpr int EPC = 32 / NQ;  // weights per QK chunk
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    const float nm = -m;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8 pb[2][2];
    bf16x8 kq[NQ];
#pragma unroll
    for (int c = 0; c < KA; ++c) kq[c] = kfrag(c);
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      if (c + KA < NQ) kq[c + KA] = kfrag(c + KA);
      sn[c & 1] = mfma_bf16(kq[c], qf[c >> 1], sn[c & 1]);
#pragma unroll
      for (int u = 0; u < EPC; ++u) {
        const int x = EPC * c + u, nt = x >> 4, r = x & 15;
        const float e = fast_exp2(__builtin_fmaf(sc[nt][r], sl2, nm));
        rs[r & 3] += e;
        pb[nt][r >> 3][r & 7] = to_bf16(e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    bf16x8 vq[NP];
#pragma unroll
    for (int c = 0; c < VA; ++c) vq[c] = vfrag(c);
    float mx0 = kNegInf, mx1 = kNegInf;
    constexpr int MPC = 32 / NP;  // row-max elements per P.V chunk
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      if (c + VA < NP) vq[c + VA] = vfrag(c + VA);
      o[c % DT] = mfma_bf16(vq[c], pb[(c / DT) >> 1][(c / DT) & 1], o[c % DT]);
#pragma unroll
      for (int u = 0; u < MPC; u += 2) {
        const int x = MPC * c + u, nt = x >> 4, r = x & 15;
        if (nt == 0) mx0 = fmaxf(mx0, fmaxf(sn[0][r], sn[0][r + 1]));
        else mx1 = fmaxf(mx1, fmaxf(sn[1][r], sn[1][r + 1]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mxn = pair_max(fmaxf(mx0, mx1)) * sl2;
  }

  template <bool MASK>
  __device__ __forceinline__ void step(const char* buf, int lane, int key0, int qpos, float sl2) {
    const int h = lane >> 5, col = lane & 31;
    f32x16 s[2] = {f32x16{}, f32x16{}};
    {
      // Rows col and 32 + col share swz (it depends on row % 16 only), so
      // one offset pattern serves both key halves.
      const int sw = swz(col);
      const char* r0 = buf + col * ROWB;
      const char* r1 = r0 + 32 * ROWB;
      bf16x8 a[KC];
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) a[kk] = *reinterpret_cast<const bf16x8*>(r0 + 16 * ((2 * kk + h) ^ sw));
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        s[0] = mfma_bf16(a[kk], qf[kk], s[0]);
        a[kk] = *reinterpret_cast<const bf16x8*>(r1 + 16 * ((2 * kk + h) ^ sw));
      }
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) s[1] = mfma_bf16(a[kk], qf[kk], s[1]);
    }
    // P.V operands: lane j of each 16-lane group names row K0 + j/4, dims
    // D0 + 4*(j%4) .. +3 and receives V[K0 + e][D0 + j], e < 4, i.e. a V^T
    // fragment.
    const int j = lane & 15, half = (lane >> 4) & 1;
    const char* vb = buf + TB;
    auto vfrag = [&](int dt, int nt, int g) {
      const int d = 32 * dt + 16 * half + 4 * (j & 3);
      const int r0 = 32 * nt + 16 * g + 4 * h + (j >> 2), r1 = r0 + 8;
      const char* a0 = vb + r0 * ROWB + 16 * ((d >> 3) ^ swzv(r0)) + 2 * (d & 7);
      const char* a1 = vb + r1 * ROWB + 16 * ((d >> 3) ^ swzv(r1)) + 2 * (d & 7);
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a1));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    online_softmax<MASK>(s, m, l, o, h, key0, qpos, sl2);
    bf16x8 pb[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) pb[nt][r >> 3][r & 7] = to_bf16(s[nt][r]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = mfma_bf16(vfrag(dt, i >> 1, i & 1), pb[i >> 1][i & 1], o[dt]);
  }

  // 16 output values of d-tile dt, lane-native order, to memory.
  static __device__ __forceinline__ void put16(bf16* dst, const f32x16& x, float scale) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = to_bf16(x[e] * scale);
      b[e] = to_bf16(x[8 + e] * scale);
    }
    *reinterpret_cast<bf16x8*>(dst) = a;
    *reinterpret_cast<bf16x8*>(dst + 8) = b;
  }
  static __device__ __forceinline__ void get16(const bf16* src, float (&x)[16]) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(src);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(src + 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = (float)a[e];
      x[8 + e] = (float)b[e];
    }
  }
  // Four consecutive output coordinates (one r-group) to o.
  static __device__ __forceinline__ void put4(bf16* dst, float a0, float a1, float a2, float a3) {
    bf16x4 v;
    v[0] = to_bf16(a0);
    v[1] = to_bf16(a1);
    v[2] = to_bf16(a2);
    v[3] = to_bf16(a3);
    *reinterpret_cast<bf16x4*>(dst) = v;
  }
};

// ------------------------------------------------------------ fp32 engine
template <int D>
struct EngF32 {
  using T = float;
  static constexpr bool kDMA = false;
  static constexpr int KC = D / 2, DT = D / 32;
  static constexpr int KS = D + 2;  // K row stride (floats): conflict-free column reads
  static constexpr int VS = D + 8;  // V row stride (floats): the two lane halves hit disjoint banks
  static constexpr int BUF_BYTES = (kSub * KS + kSub * VS) * 4;
  static constexpr int CH = kSub * D / 4;  // 16-byte chunks per subtile

  float qf[KC];
  f32x16 o[DT];
  float m, l;

  template <int NT>
  struct Stage {
    u32x4 k[(CH + NT - 1) / NT];
    u32x4 v[(CH + NT - 1) / NT];
  };

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    m = kNegInf;
    l = 0.f;
  }
  __device__ __forceinline__ void load_q(const float* qrow, int h) {
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) qf[kk] = qrow[2 * kk + h];
  }
  // Load one K and one V subtile into registers.
  template <int NT>
  static __device__ __forceinline__ void begin(Stage<NT>& st, const float* kp, const float* vp, char*, int tid) {
#pragma unroll
    for (int i = 0; i < (CH + NT - 1) / NT; ++i) {
      const int id = tid + NT * i;
      if (CH % NT == 0 || id < CH) {
        const int row = id / (D / 4), cc = id % (D / 4);
        st.k[i] = *reinterpret_cast<const u32x4*>(kp + (int64_t)row * D + 4 * cc);
        st.v[i] = *reinterpret_cast<const u32x4*>(vp + (int64_t)row * D + 4 * cc);
      }
    }
  }
  // Write the staged registers to the LDS buffer.
  template <int NT>
  static __device__ __forceinline__ void land(const Stage<NT>& st, char* buf, int tid) {
    float* Ks = reinterpret_cast<float*>(buf);
    float* Vs = Ks + kSub * KS;
#pragma unroll
    for (int i = 0; i < (CH + NT - 1) / NT; ++i) {
      const int id = tid + NT * i;
      if (CH % NT == 0 || id < CH) {
        const int row = id / (D / 4), cc = id % (D / 4);
        float* kd = Ks + row * KS + 4 * cc;
        *reinterpret_cast<u32x2*>(kd) = u32x2{st.k[i].x, st.k[i].y};
        *reinterpret_cast<u32x2*>(kd + 2) = u32x2{st.k[i].z, st.k[i].w};
        *reinterpret_cast<u32x4*>(Vs + row * VS + 4 * cc) = st.v[i];
      }
    }
  }
  template <bool MASK>
  __device__ __forceinline__ void step(const char* buf, int lane, int key0, int qpos, float sl2) {
    const int h = lane >> 5, col = lane & 31;
    const float* Ks = reinterpret_cast<const float*>(buf);
    const float* Vs = Ks + kSub * KS;
    f32x16 s[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      s[nt] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) s[nt] = mfma_f32(Ks[(32 * nt + col) * KS + 2 * kk + h], qf[kk], s[nt]);
    }
    online_softmax<MASK>(s, m, l, o, h, key0, qpos, sl2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          o[dt] = mfma_f32(Vs[(32 * nt + crow(r, h)) * VS + 32 * dt + col], s[nt][r], o[dt]);
    }
  }
  static __device__ __forceinline__ void put16(float* dst, const f32x16& x, float scale) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = x[4 * q4 + e] * scale;
      *reinterpret_cast<f32x4*>(dst + 4 * q4) = v;
    }
  }
  static __device__ __forceinline__ void get16(const float* src, float (&x)[16]) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q4 + e] = v[e];
    }
  }
  static __device__ __forceinline__ void put4(float* dst, float a0, float a1, float a2, float a3) {
    f32x4 v;
    v[0] = a0;
    v[1] = a1;
    v[2] = a2;
    v[3] = a3;
    *reinterpret_cast<f32x4*>(dst) = v;
  }
};

template <typename T, int D>
struct EngOf;
template <int D>
struct EngOf<bf16, D> {
  using type = EngBF16<D>;
};
template <int D>
struct EngOf<float, D> {
  using type = EngF32<D>;
};

// Streams nsub consecutive 64-key subtiles of K and V through LDS and calls
// compute(buf, sub) on each. Direct-load engines double-buffer (loads of
// subtile sub+1 run under the compute of subtile sub; the two buffers are
// distinct objects so the compiler need not order the loads against the
// reads of the other buffer); register-staged engines prefetch into
// registers and use one buffer.
// start() runs once the first subtile's loads are queued (work whose own
// loads should overlap them: the query rows, the merge's partials).
template <class E, int NT, class S, class F>
__device__ __forceinline__ void stream_subtiles(char* bufA, char* bufB, const typename E::T* kp,
                                                const typename E::T* vp, int nsub, int D, int tid, S&& start,
                                                F&& compute) {
  typename E::template Stage<NT> st;
  if constexpr (E::kDMA) {
    // Direct loads from wave-uniform bases with per-lane offsets computed
    // once (no per-load address arithmetic).
    typename E::template LoadOffsets<NT> lo;
    E::template load_offsets<NT>(lo, tid);
    auto issue = [&](int sub, char* buf) {
      E::template begin_uniform<NT, false>(kp + sub * (int64_t)kSub * D, lo, buf, tid);
      E::template begin_uniform<NT, true>(vp + sub * (int64_t)kSub * D, lo, buf + E::TB, tid);
    };
    issue(0, bufA);
    start();
    lds_dma_wait();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query fragments too (see below)
    __syncthreads();
    for (int sub = 0; sub < nsub; sub += 2) {
      const bool m1 = sub + 1 < nsub;
      if (m1) issue(sub + 1, bufB);
      compute(bufA, sub);
      if (m1) lds_dma_wait();
      __syncthreads();
      if (!m1) break;
      const bool m2 = sub + 2 < nsub;
      if (m2) issue(sub + 2, bufA);
      compute(bufB, sub + 1);
      if (m2) lds_dma_wait();
      __syncthreads();
    }
    return;
  }
  E::template begin<NT>(st, kp, vp, bufA, tid);
  start();
  E::template land<NT>(st, bufA, tid);
  // Also tell the compiler that every vector-memory load issued so far (the
  // query fragments) has completed, so that it emits no vmcnt waits inside
  // the loop, where the only outstanding loads are the next subtile's.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  const int64_t step_elems = (int64_t)kSub * D;
  if constexpr (E::kDMA) {
    for (int sub = 0; sub < nsub; sub += 2) {
      const bool m1 = sub + 1 < nsub;
      if (m1) E::template begin<NT>(st, kp + (sub + 1) * step_elems, vp + (sub + 1) * step_elems, bufB, tid);
      compute(bufA, sub);
      if (m1) E::template land<NT>(st, bufB, tid);
      __syncthreads();
      if (!m1) break;
      const bool m2 = sub + 2 < nsub;
      if (m2) E::template begin<NT>(st, kp + (sub + 2) * step_elems, vp + (sub + 2) * step_elems, bufA, tid);
      compute(bufB, sub + 1);
      if (m2) E::template land<NT>(st, bufA, tid);
      __syncthreads();
    }
  } else {
    for (int sub = 0; sub < nsub; ++sub) {
      const bool more = sub + 1 < nsub;
      if (more) E::template begin<NT>(st, kp + (sub + 1) * step_elems, vp + (sub + 1) * step_elems, bufA, tid);
      compute(bufA, sub);
      if (more) {
        __syncthreads();
        E::template land<NT>(st, bufA, tid);
      }
      __syncthreads();
    }
  }
}

// K-ahead stream for direct-load engines, unmasked subtiles only (gather):
// each buffer holds a K subtile then a V subtile (TB bytes each). Step sub
// loads K of sub+2 and V of sub+1, computes the scores of sub+1 while the
// weights and P.V of sub run, and ends at the barrier that publishes the
// loads. Buffer use: K(sub) in buf[sub % 2], V(sub) in buf[sub % 2] + TB;
// K(sub+2) overwrites K(sub), read in the step before (or the prologue,
// followed by its own barrier), V(sub+1) overwrites V(sub-1), read in the
// step before.
template <class E, int NT, bool ON, class S>
__device__ __forceinline__ void stream_k_ahead_t(E& eng, char* bufA, char* bufB, const typename E::T* kp,
                                                 const typename E::T* vp, int nsub, int tid, int lane, float sl2,
                                                 S&& start) {
  constexpr int64_t SE = (int64_t)kSub * E::kD;
  typename E::template LoadOffsets<NT> lo;
  E::template load_offsets<NT>(lo, tid);
  E::template begin_uniform<NT, false>(kp, lo, bufA, tid);
  E::template begin_uniform<NT, true>(vp, lo, bufA + E::TB, tid);
  if (nsub > 1) E::template begin_uniform<NT, false>(kp + SE, lo, bufB, tid);
  start();  // e.g. the query rows, under the first K/V loads
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): see stream_subtiles
  lds_dma_wait();
  __syncthreads();
  f32x16 sa[2], sb[2];
  float ma = kNegInf, mb = kNegInf;
  if (ON) {
    eng.qk(bufA, lane, sa);
    ma = E::rowmax(sa, sl2);
  }
  __syncthreads();
  // A step with a next subtile (its scores are computed here). Both loads
  // it queues are read by the very next step (K(sub+2) for that step's
  // scores, V(sub+1) for its P.V), so the step ends waiting for all of this
  // wave's loads before the barrier that publishes them to the other waves.
  auto full = [&](int sub, char* bc, char* bn, f32x16(&sc)[2], f32x16(&sn)[2], float mc, float& mn) {
    const bool k2 = sub + 2 < nsub;
    E::template begin_uniform<NT, true>(vp + (sub + 1) * SE, lo, bn + E::TB, tid);
    if (k2) E::template begin_uniform<NT, false>(kp + (sub + 2) * SE, lo, bc, tid);
    if (ON) {
      eng.rescale(mc);
      eng.fused(bn, sn, sc, bc + E::TB, lane, sl2, mn);
    }
    lds_dma_wait();
    __syncthreads();
  };
  // The final step.
  auto last = [&](char* bc, f32x16(&sc)[2], float mc) {
    if (ON) {
      eng.rescale(mc);
      eng.expo_pv(sc, bc + E::TB, lane, sl2);
    }
  };
  int sub = 0;
  for (; sub + 2 < nsub; sub += 2) {
    full(sub, bufA, bufB, sa, sb, ma, mb);
    full(sub + 1, bufB, bufA, sb, sa, mb, ma);
  }
  if (sub + 1 < nsub) {
    full(sub, bufA, bufB, sa, sb, ma, mb);
    last(bufB, sb, mb);
  } else {
    last(bufA, sa, ma);
  }
}

// K-ahead stream (see stream_k_ahead_t); waves without queries (on false)
// take part in the loads and barriers only.
template <class E, int NT, class S>
__device__ __forceinline__ void stream_k_ahead(E& eng, char* bufA, char* bufB, const typename E::T* kp,
                                               const typename E::T* vp, int nsub, int tid, int lane, bool on,
                                               float sl2, S&& start) {
  if (on) stream_k_ahead_t<E, NT, true>(eng, bufA, bufB, kp, vp, nsub, tid, lane, sl2, start);
  else stream_k_ahead_t<E, NT, false>(eng, bufA, bufB, kp, vp, nsub, tid, lane, sl2, start);
}

// LDS for one kernel: two static subtile buffers for direct-load engines,
// the dynamic allocation (one buffer) otherwise.
#define MOBA_KERNEL_LDS(E)                                                   \
  extern __shared__ __align__(16) char dyn_smem[];                           \
  __shared__ __align__(16) char lds_a[E::kDMA ? E::BUF_BYTES : 16];          \
  __shared__ __align__(16) char lds_b[E::kDMA ? E::BUF_BYTES : 16];          \
  char* bufA = E::kDMA ? lds_a : dyn_smem;                                   \
  char* bufB = E::kDMA ? lds_b : dyn_smem;

template <class E>
constexpr int dyn_lds_bytes() {
  return E::kDMA ? 0 : E::BUF_BYTES;
}

}  // namespace

// ------------------------------------------------------- past-block gather
template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void gather_attn_kernel(AttnArgs a) {
  using E = typename EngOf<T, D>::type;
  constexpr int NT = 64 * NW;
  MOBA_KERNEL_LDS(E)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;

  // This workgroup's tile: its (head, block) and list range (written by the
  // packing step, which also spreads tiles over the XCDs).
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 tm = *reinterpret_cast<const i32x4*>(a.tile_map + 4 * (int64_t)blockIdx.x);
  if (tm.x < 0) return;
  const int64_t blk = __builtin_amdgcn_readfirstlane(tm.x);  // uniform: keeps the K/V bases in SGPRs
  const int64_t bh = blk / a.n_blocks, j = blk % a.n_blocks;
  const int64_t e0 = __builtin_amdgcn_readfirstlane(tm.y), e1 = __builtin_amdgcn_readfirstlane(tm.z);
  const int64_t e = e0 + 32 * w + col;
  const bool valid = e < e1;
  const bool wave_on = e0 + 32 * w < e1;
  const int slots = a.k_eff - 1;
  int ev = 0, t = 0;

  E eng;
  eng.init();
  const T* q = reinterpret_cast<const T*>(a.q);
  // Query rows: read after the first K/V loads are queued.
  auto load_q = [&]() {
    ev = a.qlist[valid ? e : e0];
    t = ev / slots;
    if (wave_on) eng.load_q(q + (bh * a.seq_len + t) * D, h);
  };
  // Keys and values of the query head's key/value head (grouped-query attention).
  const int64_t kvh = bh / a.group;
  const T* kp = reinterpret_cast<const T*>(a.k) + (kvh * a.seq_len + j * a.block_size) * D;
  const T* vp = reinterpret_cast<const T*>(a.v) + (kvh * a.seq_len + j * a.block_size) * D;
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  // A short last block (seq_len not a multiple of block_size) has fewer subtiles.
  const int nsub = (int)(min<int64_t>(a.block_size, a.seq_len - j * a.block_size) / kSub);
  if constexpr (E::kDMA) {
    stream_k_ahead<E, NT>(eng, bufA, bufB, kp, vp, nsub, tid, lane, wave_on, sl2, load_q);
  } else {
    stream_subtiles<E, NT>(bufA, bufB, kp, vp, nsub, D, tid, load_q, [&](const char* buf, int) {
      if (wave_on) eng.template step<false>(buf, lane, 0, 0, sl2);
    });
  }
  if (!wave_on) return;
  const float lt = pair_sum(eng.l);
  if (valid) {
    const int64_t rec = bh * a.seq_len * slots + ev;
    T* dst = reinterpret_cast<T*>(a.part_o) + rec * D + h * (D / 2);
    const float inv = 1.f / lt;
#pragma unroll
    for (int dt = 0; dt < E::DT; ++dt) E::put16(dst + 16 * dt, eng.o[dt], inv);
    if (h == 0) a.part_lse[rec] = eng.m + fast_log2(lt);
  }
}

// --------------------------------------------- own block + merge (and dense)
template <typename T, int D, int NW, bool DENSE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void diag_attn_kernel(AttnArgs a) {
  using E = typename EngOf<T, D>::type;
  constexpr int NT = 64 * NW, M = 32 * NW;
  MOBA_KERNEL_LDS(E)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  // Heavier tiles (later in the sequence) first, heads interleaved.
  const int64_t ntile = a.seq_len / M;
  const int64_t tile = ntile - 1 - blockIdx.x / a.bh;
  const int64_t bh = blockIdx.x % a.bh;
  const int q0 = (int)(tile * M);
  const int c = (int)(q0 / a.block_size);
  const int kb = DENSE ? 0 : (int)(c * a.block_size);
  const int kend = a.causal ? q0 + M : (DENSE ? (int)a.seq_len : (int)min<int64_t>(kb + a.block_size, a.seq_len));
  const int qw0 = q0 + 32 * w;
  const int t = qw0 + col;

  E eng;
  eng.init();
  const T* q = reinterpret_cast<const T*>(a.q);
  // Query rows, and for the own block the merge's seed: run once the first
  // K/V loads are queued, so that their loads overlap.
  auto start = [&]() {
    eng.load_q(q + (bh * a.seq_len + t) * D, h);
    if (DENSE) return;
    // Start the online softmax from the past-block partials: with
    // m = max lse_i and w_i = 2^(lse_i - m), the state (m, sum w_i,
    // sum w_i o_i) is the partials' union, and the own block's keys then
    // continue it, so the merge needs no pass after the loop. l is kept on
    // one lane of the pair, which sums it at the end.
    const int n_elig = a.causal ? c : (int)a.n_blocks - 1;
    const int n = min(a.k_eff - 1, n_elig);
    const int slots = a.k_eff - 1;
    const int64_t rec0 = (bh * a.seq_len + t) * (int64_t)slots;
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
  const int64_t kvh = bh / a.group;  // the query head's key/value head
  const T* kp = reinterpret_cast<const T*>(a.k) + (kvh * a.seq_len + kb) * D;
  const T* vp = reinterpret_cast<const T*>(a.v) + (kvh * a.seq_len + kb) * D;
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int nsub = (kend - kb) / kSub;
  // Subtiles entirely before the workgroup's first query need no mask; with
  // causal attention the last M/64 subtiles hold the diagonal.
  const int nfree = a.causal ? (q0 - kb) / kSub : nsub;
  stream_subtiles<E, NT>(bufA, bufB, kp, vp, nsub, D, tid, start, [&](const char* buf, int sub) {
    if (sub < nfree) {
      eng.template step<false>(buf, lane, 0, 0, sl2);
    } else {
      const int key0 = kb + sub * kSub;
      // Skip a subtile whose keys all come after every query of this wave.
      if (key0 <= qw0 + 31) eng.template step<true>(buf, lane, key0, t, sl2);
    }
  });

  // Dense, or own block continuing the partials' state: normalise once.
  const float lt = pair_sum(eng.l);
  const float inv = 1.f / lt;
  // The natural-log log-sum-exp of the query's scaled logits over every key
  // it attended (m and l are in the log2 domain), for a backward pass.
  if (a.lse_out && h == 0) a.lse_out[bh * a.seq_len + t] = (eng.m + fast_log2(lt)) * 0.69314718f;
#pragma unroll
  for (int dt = 0; dt < E::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) eng.o[dt][r] *= inv;
  T* orow = reinterpret_cast<T*>(a.o) + (bh * a.seq_len + t) * D;
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
  // 128-query tiles when they stay inside one block (and one sequence), else 64.
  const bool four = a.seq_len % 128 == 0 && (DENSE || a.block_size % 128 == 0);
  const char* name = DENSE ? "dense_attn" : "diag_merge";
  constexpr int lds = dyn_lds_bytes<E>();
  if (four) {
    auto kern = diag_attn_kernel<T, D, 4, DENSE>;
    hipError_t e = prep_lds(kern, lds);
    if (e != hipSuccess) return e;
    KernelTimer timer(s, name);
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.bh * (a.seq_len / 128))), dim3(256), lds, s, a);
  } else {
    auto kern = diag_attn_kernel<T, D, 2, DENSE>;
    hipError_t e = prep_lds(kern, lds);
    if (e != hipSuccess) return e;
    KernelTimer timer(s, name);
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.bh * (a.seq_len / 64))), dim3(128), lds, s, a);
  }
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


// ================================================================ backward
// MoBA backward for bf16 inputs, the block choice of the forward held fixed
// (a top-k over block scores has no gradient off ties, and the gate's
// scores do not weight the output): per query, the gradient of one softmax
// attention over its attended keys. With l = q.k / sqrt(D), p = exp(l - lse),
// delta = do . o:  dv_u += p_u do,  ds_u = p_u (do . v_u - delta),
// dq += ds_u k_u / sqrt(D),  dk_u += ds_u q / sqrt(D).
//
// Kernels (each step single-buffered: load a 64-row subtile to LDS, wait,
// compute, barrier):
//  bwd_prep    — delta and the log-sum-exp in the log2 domain per query;
//  dq_past     — block-major like gather_attn (the forward's lists and
//                tiles): per key subtile S^T = K Q^T and dP^T = V dO^T on
//                the forward's score path, then dQ^T += K^T dS^T on its P.V
//                path (the same K copy read through the LDS transpose
//                load); subtiles double-buffered; one fp32
//                partial per (query, slot);
//  dq_own      — the own block, 64 queries per workgroup, causal mask; it
//                then adds the slots' partials in slot order and writes dq
//                (no atomics);
//  dkv         — key-major: a workgroup holds 128 (or 64) keys of one
//                block (32 per wave, as the B operand the way the forward
//                holds queries)
//                and streams 64-row subtiles of the queries that attend
//                them: the block's own queries, then its listed queries
//                (gathered rows), for every query head of the key/value
//                head. PASS 0 accumulates dV^T += dO^T P, PASS 1
//                dK^T += Q^T dS (both on the P.V path); together they would
//                not fit the register file.
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
template <int D, bool VSW = true>
__device__ __forceinline__ void mm_trans(const char* buf, int lane, const f32x16 (&x)[2], f32x16 (&acc)[D / 32]) {
  using E = EngBF16<D>;
  const int h = lane >> 5, j = lane & 15, half = (lane >> 4) & 1;
  bf16x8 pb[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) pb[nt][r >> 3][r & 7] = to_bf16(x[nt][r]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int nt = i >> 1, g = i & 1;
      const int d = 32 * dt + 16 * half + 4 * (j & 3);
      const int r0 = 32 * nt + 16 * g + 4 * h + (j >> 2), r1 = r0 + 8;
      const int s0 = VSW ? E::swzv(r0) : E::swz(r0), s1 = VSW ? E::swzv(r1) : E::swz(r1);
      const char* a0 = buf + r0 * E::ROWB + 16 * ((d >> 3) ^ s0) + 2 * (d & 7);
      const char* a1 = buf + r1 * E::ROWB + 16 * ((d >> 3) ^ s1) + 2 * (d & 7);
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a1));
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[dt] = mfma_bf16(vf, pb[nt][g], acc[dt]);
    }
}

// A row's D/16 B fragments for this lane half (like EngBF16::load_q).
template <int D>
__device__ __forceinline__ void load_frags(bf16x8 (&f)[D / 16], const bf16* row, int h) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = *reinterpret_cast<const bf16x8*>(row + 16 * kk + 8 * h);
}

// acc (C layout of mm_trans: lane column = row of dst, element r = coordinate
// 32 dt + crow(r, h)) times scale, to a row of dst in fp32 or bf16.
template <int D>
__device__ __forceinline__ void store_row_f32(float* dst, const f32x16 (&acc)[D / 32], int h, float scale) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      *reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * rg + 4 * h) =
          f32x4{acc[dt][4 * rg] * scale, acc[dt][4 * rg + 1] * scale, acc[dt][4 * rg + 2] * scale,
                acc[dt][4 * rg + 3] * scale};
}
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
template <int D>
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
  const int ev = a.qlist[valid ? e : e0];
  const int t = ev / slots;
  const int64_t row = bh * a.seq_len + t;
  bf16x8 qf[KC], gf[KC];
  load_frags<D>(qf, reinterpret_cast<const bf16*>(a.q) + row * D, h);
  load_frags<D>(gf, reinterpret_cast<const bf16*>(a.dout) + row * D, h);
  const float lse2 = a.lse2[row], delta = a.delta[row];
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int64_t kvh = bh / a.group;
  const bf16* kp = reinterpret_cast<const bf16*>(a.k) + (kvh * a.seq_len + j * a.block_size) * D;
  const bf16* vp = reinterpret_cast<const bf16*>(a.v) + (kvh * a.seq_len + j * a.block_size) * D;
  const int nsub = (int)(min<int64_t>(a.block_size, a.seq_len - j * a.block_size) / kSub);
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  // Double-buffered: the loads of subtile sub + 1 run under the compute of
  // sub (buffer sub & 1); each step ends waiting for them, then the barrier.
  E::template begin_one<NT, false>(kp, bk0, tid);
  E::template begin_one<NT, false>(vp, bv0, tid);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), also for the query rows
  lds_dma_wait();
  __syncthreads();
  for (int sub = 0; sub < nsub; ++sub) {
    const bool odd = sub & 1;
    if (sub + 1 < nsub) {
      E::template begin_one<NT, false>(kp + (int64_t)(sub + 1) * kSub * D, odd ? bk0 : bk1, tid);
      E::template begin_one<NT, false>(vp + (int64_t)(sub + 1) * kSub * D, odd ? bv0 : bv1, tid);
    }
    if (wave_on) dq_step<D, false>(odd ? bk1 : bk0, odd ? bv1 : bv0, lane, qf, gf, lse2, delta, sl2, 0, 0, acc);
    lds_dma_wait();
    __syncthreads();
  }
  if (valid) store_row_f32<D>(a.dq_part + ((bh * a.seq_len * slots) + ev) * D, acc, h, 1.f / __builtin_sqrtf((float)D));
}

// The own block: 64 consecutive queries of one head.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void dq_own_kernel(BwdArgs a) {
  using E = EngBF16<D>;
  constexpr int NT = 64 * NW, KC = D / 16, DT = D / 32, M = 32 * NW;
  // Single-buffered (32 KB), so that several workgroups share a compute unit.
  __shared__ __align__(16) char bk[E::TB], bv[E::TB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  const int64_t ntile = a.seq_len / M;
  const int64_t bh = blockIdx.x / ntile;
  const int q0 = (int)((blockIdx.x % ntile) * M);
  const int c = (int)(q0 / a.block_size);
  const int kb = (int)(c * a.block_size);
  const int kend = a.causal ? q0 + M : (int)min<int64_t>(kb + a.block_size, a.seq_len);
  const int t = q0 + 32 * w + col;
  const int64_t row = bh * a.seq_len + t;
  bf16x8 qf[KC], gf[KC];
  load_frags<D>(qf, reinterpret_cast<const bf16*>(a.q) + row * D, h);
  load_frags<D>(gf, reinterpret_cast<const bf16*>(a.dout) + row * D, h);
  const float lse2 = a.lse2[row], delta = a.delta[row];
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int64_t kvh = bh / a.group;
  const bf16* kp = reinterpret_cast<const bf16*>(a.k) + (kvh * a.seq_len + kb) * D;
  const bf16* vp = reinterpret_cast<const bf16*>(a.v) + (kvh * a.seq_len + kb) * D;
  const int nsub = (kend - kb) / kSub;
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  for (int sub = 0; sub < nsub; ++sub) {
    E::template begin_one<NT, false>(kp + (int64_t)sub * kSub * D, bk, tid);
    E::template begin_one<NT, false>(vp + (int64_t)sub * kSub * D, bv, tid);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), also for the query rows
    lds_dma_wait();
    __syncthreads();
    const int key0 = kb + sub * kSub;
    if (a.causal && key0 + kSub > q0 + 32 * w) {
      if (key0 <= q0 + 32 * w + 31) dq_step<D, true>(bk, bv, lane, qf, gf, lse2, delta, sl2, key0, t, acc);
    } else {
      dq_step<D, false>(bk, bv, lane, qf, gf, lse2, delta, sl2, 0, 0, acc);
    }
    __syncthreads();
  }
  // dq = own-block part + the past slots' partials (written by dq_past, an
  // earlier launch) in slot order, rounded once to bf16.
  const float scale = 1.f / __builtin_sqrtf((float)D);
  const int n_elig = a.causal ? c : (int)a.n_blocks - 1;
  const int slots = a.k_eff - 1;
  const int n = min(slots, n_elig);
  bf16* dst = reinterpret_cast<bf16*>(a.dq) + row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = 32 * dt + 8 * rg + 4 * h;
      f32x4 x = f32x4{acc[dt][4 * rg] * scale, acc[dt][4 * rg + 1] * scale, acc[dt][4 * rg + 2] * scale,
                      acc[dt][4 * rg + 3] * scale};
      for (int sl = 0; sl < n; ++sl) x += *reinterpret_cast<const f32x4*>(a.dq_part + (row * slots + sl) * D + d);
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
    const int t = a.qlist[pos] / slots;
    a.lt[pos] = t;
    a.ll[pos] = a.lse2[bh * a.seq_len + t];
    a.ld[pos] = a.delta[bh * a.seq_len + t];
  }
}

// dV (PASS 0; dK is dk_kernel) for 32 * NW keys of one block of one
// key/value head. The 64-row query subtiles that attend those keys (for
// every query head of the group: the block's own queries at or after the
// keys, then its listed queries) are numbered 0 .. N-1 and software
// pipelined over two LDS buffer sets: while subtile i is computed from one
// set, the rows of i + 1 load into the other, and wave 0 holds the row
// numbers, log-sum-exps and deltas of i + 2 in registers. Q and dO are
// staged once each (K-swizzled); the dK and dV products read them
// transposed from the same copy.
template <int D, int PASS, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void dkv_kernel(BwdArgs a) {
  using E = EngBF16<D>;
  constexpr int NT = 64 * NW, KC = D / 16, DT = D / 32, KEYS = 32 * NW;
  __shared__ __align__(16) char bq[2][E::TB], bx[2][E::TB];
  __shared__ int rows[2][64];
  __shared__ float lse2s[2][64], deltas[2][64];
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
  const int u = (int)k0 + 32 * w + col;  // this lane's key
  const bf16* krow = reinterpret_cast<const bf16*>(a.k) + (kvh * a.seq_len + u) * D;
  const bf16* vrow = reinterpret_cast<const bf16*>(a.v) + (kvh * a.seq_len + u) * D;
  bf16x8 kf[KC], vf[PASS == 1 ? KC : 1];
  load_frags<D>(kf, krow, h);
  if constexpr (PASS == 1) load_frags<D>(vf, vrow, h);
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int slots = a.k_eff - 1;
  const int64_t jend = min<int64_t>((j + 1) * a.block_size, a.seq_len);
  const int64_t qs = a.causal ? k0 : j * a.block_size;  // first own query that sees the keys
  const int n_own = (int)((jend - qs + 63) / 64);
  // Subtile i: (query head, own or listed, first row or list position, rows).
  struct Sub {
    int64_t bh;
    int64_t first;
    int n;
    bool own;
  };
  auto sub_at = [&](int i) {
    Sub d{};
    for (int g = 0; g < a.group; ++g) {
      const int64_t bh = kvh * a.group + g;
      if (i < n_own) {
        d.bh = bh;
        d.own = true;
        d.first = qs + 64 * (int64_t)i;
        d.n = (int)min<int64_t>(64, jend - d.first);
        return d;
      }
      i -= n_own;
      int64_t o0 = 0, cnt = 0;
      if (slots > 0) {
        o0 = a.offset[bh * a.n_blocks + j];
        cnt = a.offset[bh * a.n_blocks + j + 1] - o0;
      }
      const int n_list = (int)((cnt + 63) / 64);
      if (i < n_list) {
        d.bh = bh;
        d.own = false;
        d.first = o0 + 64 * (int64_t)i;
        d.n = (int)min<int64_t>(64, cnt - 64 * (int64_t)i);
        return d;
      }
      i -= n_list;
    }
    return d;
  };
  int total = 0;
  for (int g = 0; g < a.group; ++g) {
    const int64_t bh = kvh * a.group + g;
    int64_t cnt = 0;
    if (slots > 0) cnt = a.offset[bh * a.n_blocks + j + 1] - a.offset[bh * a.n_blocks + j];
    total += n_own + (int)((cnt + 63) / 64);
  }
  // Wave 0's registers: row number, log-sum-exp and delta of its lane's row
  // of a subtile (a padding row repeats the first row with weight 0).
  int mt = 0;
  float ml = 0.f, md = 0.f;
  auto meta_load = [&](const Sub& d) {
    const bool ok = lane < d.n;
    const int64_t i = d.first + (ok ? lane : 0);
    if (d.own) {
      mt = (int)i;
      ml = a.lse2[d.bh * a.seq_len + i];
      md = a.delta[d.bh * a.seq_len + i];
    } else {
      mt = a.lt[i];
      ml = a.ll[i];
      md = a.ld[i];
    }
    if (!ok) {
      ml = __builtin_inff();
      md = 0.f;
    }
  };
  auto meta_store = [&](int x) {
    rows[x][lane] = mt;
    lse2s[x][lane] = ml;
    deltas[x][lane] = md;
  };
  auto rows_in = [&](const Sub& d, int x) {
    const bf16* qb = reinterpret_cast<const bf16*>(a.q) + d.bh * a.seq_len * D;
    const bf16* gb = reinterpret_cast<const bf16*>(a.dout) + d.bh * a.seq_len * D;
    load_rows<D, NT, false>(qb, rows[x], bq[x], tid);
    load_rows<D, NT, false>(gb, rows[x], bx[x], tid);
  };
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  auto compute = [&](const Sub& d, int x) {
    const bool mask = d.own && a.causal;
    f32x16 s[2];
    mm_rows<D>(bq[x], lane, kf, s);
    f32x16 dp[2];
    if constexpr (PASS == 1) mm_rows<D>(bx[x], lane, vf, dp);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int r0 = 32 * nt + 8 * rg + 4 * h;  // rows of elements 4 rg .. 4 rg + 3
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[x][r0]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&deltas[x][r0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          float p = fast_exp2(__builtin_fmaf(s[nt][r], sl2, -l4[e]));
          if (mask && u > rows[x][r0 + e]) p = 0.f;
          if constexpr (PASS == 0) s[nt][r] = p;
          else s[nt][r] = p * (dp[nt][r] - d4[e]);
        }
      }
    // dV^T += dO^T P or dK^T += Q^T dS, read transposed from the K-swizzled copy.
    mm_trans<D, false>(PASS == 0 ? bx[x] : bq[x], lane, s, acc);
  };
  // Prologue: metadata of 0 stored, rows of 0 loading, metadata of 1 in
  // wave 0's registers.
  Sub cur = sub_at(0);
  if (w == 0) {
    meta_load(cur);
    meta_store(0);
  }
  __syncthreads();
  rows_in(cur, 0);
  Sub nxt = total > 1 ? sub_at(1) : Sub{};
  if (w == 0 && total > 1) meta_load(nxt);
  for (int i = 0; i < total; ++i) {
    const int x = i & 1;
    // Wave 0 publishes the metadata of i + 1, requested during step i - 1
    // (set x ^ 1 was last read by step i - 1, before its closing barrier).
    if (w == 0 && i + 1 < total) meta_store(x ^ 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the rows of i, loaded during step i - 1
    lds_dma_wait();
    __syncthreads();
    // Under the compute of i: the rows of i + 1 and the metadata of i + 2.
    Sub nn{};
    if (i + 2 < total) nn = sub_at(i + 2);
    if (i + 1 < total) rows_in(nxt, x ^ 1);
    if (w == 0 && i + 2 < total) meta_load(nn);
    compute(cur, x);
    __syncthreads();  // set x is free for step i + 1's metadata and rows
    cur = nxt;
    nxt = nn;
  }
  bf16* dst = reinterpret_cast<bf16*>(PASS == 0 ? a.dv : a.dk) + (kvh * a.seq_len + u) * D;
  store_row_bf16<D>(dst, acc, h, PASS == 0 ? 1.f : 1.f / __builtin_sqrtf((float)D));
}

// dK (launched with PASS = 1; PASS = 0 would give dV) for 32 * NW keys of
// one block of one key/value head, single-buffered: each 64-row query
// subtile is staged (row numbers, log-sum-exps, deltas, then the rows of
// Q, dO and Q^T) and then computed. For dK this beats the pipelined
// dkv_kernel, which spills registers in this pass (same-box A/B at
// headline_32k: 1.75-1.79 against 1.94 ms; for dV the pipelined kernel
// wins, 1.47 against 1.49-1.54 ms).
template <int D, int PASS, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void dk_kernel(BwdArgs a) {
  using E = EngBF16<D>;
  constexpr int NT = 64 * NW, KC = D / 16, DT = D / 32, KEYS = 32 * NW;
  __shared__ __align__(16) char bq[E::TB], bx[E::TB], by[PASS == 1 ? E::TB : 16];
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
  const int u = (int)k0 + 32 * w + col;  // this lane's key
  const bf16* krow = reinterpret_cast<const bf16*>(a.k) + (kvh * a.seq_len + u) * D;
  const bf16* vrow = reinterpret_cast<const bf16*>(a.v) + (kvh * a.seq_len + u) * D;
  bf16x8 kf[KC], vf[PASS == 1 ? KC : 1];
  load_frags<D>(kf, krow, h);
  if constexpr (PASS == 1) load_frags<D>(vf, vrow, h);
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int slots = a.k_eff - 1;
  const int64_t jend = min<int64_t>((j + 1) * a.block_size, a.seq_len);
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  // One 64-row subtile of query head bh: rows from row_of(i) (valid when
  // i < n), causal mask against the keys when MASK.
  auto subtile = [&](int64_t bh, int n, bool mask, auto&& row_of) {
    if (tid < 64) {
      const bool ok = tid < n;
      const int t = row_of(ok ? tid : 0);  // a padding row repeats a valid one
      rows[tid] = t;
      lse2s[tid] = ok ? a.lse2[bh * a.seq_len + t] : __builtin_inff();
      deltas[tid] = ok ? a.delta[bh * a.seq_len + t] : 0.f;
    }
    __syncthreads();
    const bf16* qb = reinterpret_cast<const bf16*>(a.q) + bh * a.seq_len * D;
    const bf16* gb = reinterpret_cast<const bf16*>(a.dout) + bh * a.seq_len * D;
    load_rows<D, NT, false>(qb, rows, bq, tid);
    if constexpr (PASS == 0) {
      load_rows<D, NT, true>(gb, rows, bx, tid);   // dO^T for dV
    } else {
      load_rows<D, NT, false>(gb, rows, bx, tid);  // dO for dP
      load_rows<D, NT, true>(qb, rows, by, tid);   // Q^T for dK
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
    mm_trans<D>(PASS == 0 ? bx : by, lane, s, acc);
    __syncthreads();
  };
  for (int g = 0; g < a.group; ++g) {
    const int64_t bh = kvh * a.group + g;
    // The block's own queries: those at or after the keys (causal), or all.
    const int64_t qs = a.causal ? k0 : j * a.block_size;
    for (int64_t t0 = qs; t0 < jend; t0 += 64) {
      const int n = (int)min<int64_t>(64, jend - t0);
      subtile(bh, n, a.causal, [&](int i) { return (int)(t0 + i); });
    }
    // Its listed queries (past-block routing of later, or other, queries).
    if (slots > 0) {
      const int32_t* lst = a.qlist + a.offset[bh * a.n_blocks + j];
      const int cnt = a.offset[bh * a.n_blocks + j + 1] - a.offset[bh * a.n_blocks + j];
      for (int i0 = 0; i0 < cnt; i0 += 64) {
        const int n = min(64, cnt - i0);
        subtile(bh, n, false, [&](int i) { return lst[i0 + i] / slots; });
      }
    }
  }
  bf16* dst = reinterpret_cast<bf16*>(PASS == 0 ? a.dv : a.dk) + (kvh * a.seq_len + u) * D;
  store_row_bf16<D>(dst, acc, h, PASS == 0 ? 1.f : 1.f / __builtin_sqrtf((float)D));
}

template <int D>
hipError_t backward_t(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = a.bh * a.seq_len;
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
    hipLaunchKernelGGL(dq_past_kernel<D>, dim3((unsigned)a.gather_grid), dim3(256), 0, s, a);
  }
  {
    KernelTimer t(s, "bwd_dq_own");
    // 128 queries per workgroup where tiles of 128 stay inside one block.
    if (a.seq_len % 128 == 0 && a.block_size % 128 == 0)
      hipLaunchKernelGGL((dq_own_kernel<D, 4>), dim3((unsigned)(a.bh * (a.seq_len / 128))), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((dq_own_kernel<D, 2>), dim3((unsigned)(a.bh * (a.seq_len / 64))), dim3(128), 0, s, a);
  }
  // 128 keys per workgroup where every block length is a multiple of 128,
  // else 64.
  const int64_t last = a.seq_len - (a.n_blocks - 1) * a.block_size;
  const bool wide = a.block_size % 128 == 0 && last % 128 == 0;
  const int64_t kv_wgs = (a.bh / a.group) * a.n_blocks * (a.block_size / (wide ? 128 : 64));
  {
    KernelTimer t(s, "bwd_dv");
    if (wide) hipLaunchKernelGGL((dkv_kernel<D, 0, 4>), dim3((unsigned)kv_wgs), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dkv_kernel<D, 0, 2>), dim3((unsigned)kv_wgs), dim3(128), 0, s, a);
  }
  {
    KernelTimer t(s, "bwd_dk");
    if (wide) hipLaunchKernelGGL((dk_kernel<D, 1, 4>), dim3((unsigned)kv_wgs), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dk_kernel<D, 1, 2>), dim3((unsigned)kv_wgs), dim3(128), 0, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? backward_t<128>(a, s) : backward_t<64>(a, s);
}

}  // namespace moba
