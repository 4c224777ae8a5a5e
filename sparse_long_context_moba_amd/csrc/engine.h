// The MFMA attention engine shared by the forward (attn.hip) and the
// backward (bwd.hip): operand layouts in LDS (XOR swizzles), direct
// HBM -> LDS subtile loads, the bf16 and fp32 score / online-softmax /
// P.V steps and the subtile streams. Everything is in an anonymous
// namespace: each translation unit that includes it gets its own copy.
#pragma once
#include <type_traits>

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
  // The same offsets for a subtile holding only nrows (< 64) rows, the last
  // of a block or sequence of any length: rows at or past nrows read row
  // nrows - 1 instead (keeping the swizzle of their own LDS row), so no load
  // leaves the block; the scores of those rows are masked by the caller.
  template <int NT>
  static __device__ __forceinline__ void load_offsets_tail(LoadOffsets<NT>& lo, int tid, int nrows) {
    constexpr int NW = NT / 64;
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int ii = 0; ii < kLoadsPerWave<NT>; ++ii) {
      const int sl = (ii * NW + w) * 64 + lane, row = sl / CPR, rs = min(row, nrows - 1);
      lo.k[ii] = (unsigned)(rs * D + 8 * ((sl % CPR) ^ swz(row))) * 2u;
      lo.v[ii] = (unsigned)(rs * D + 8 * ((sl % CPR) ^ swzv(row))) * 2u;
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
  // The same loads for K or V alone, into a buffer of TB bytes, from the
  // wave-uniform base p with 32-bit lane offsets; rows at or past nrows (a
  // partial last subtile) repeat row nrows - 1.
  template <int NT, bool IS_V>
  static __device__ __forceinline__ void begin_one(const bf16* p, char* buf, int tid, int nrows = kSub) {
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
      lds_dma16_s(p, (unsigned)(min(row, nrows - 1) * D + 8 * x) * 2u, base + i * 1024);
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
  // Load one K and one V subtile into registers; a subtile holding only
  // rows (< 64) rows reads row rows - 1 for the others (their scores are
  // masked by the caller).
  template <int NT>
  static __device__ __forceinline__ void begin(Stage<NT>& st, const float* kp, const float* vp, char*, int tid,
                                               int rows) {
#pragma unroll
    for (int i = 0; i < (CH + NT - 1) / NT; ++i) {
      const int id = tid + NT * i;
      if (CH % NT == 0 || id < CH) {
        const int row = min(id / (D / 4), rows - 1), cc = id % (D / 4);
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

// The direct loads of one K (IS_V false) or V subtile holding `rows` rows
// (64, or fewer for the last subtile of a block or sequence).
template <class E, int NT, bool IS_V>
__device__ __forceinline__ void load_subtile(const typename E::T* p, const typename E::template LoadOffsets<NT>& lo,
                                             char* buf, int tid, int rows) {
  if (rows < kSub) {
    typename E::template LoadOffsets<NT> lt;
    E::template load_offsets_tail<NT>(lt, tid, rows);
    E::template begin_uniform<NT, IS_V>(p, lt, buf, tid);
  } else {
    E::template begin_uniform<NT, IS_V>(p, lo, buf, tid);
  }
}

// Scores of keys at or past nvalid in a 64-key subtile set to -inf (the
// padding rows of a partial last subtile; key 32 * nt + crow(r, h)).
__device__ __forceinline__ void mask_rows(f32x16 (&s)[2], int nvalid, int h) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * nt + crow(r, h) >= nvalid) s[nt][r] = kNegInf;
}

// Streams nsub consecutive 64-key subtiles of K and V through LDS and calls
// compute(buf, sub) on each; the last subtile holds last_rows (1..64) rows
// (the others are padding the caller masks). Direct-load engines
// double-buffer (loads of subtile sub+1 run under the compute of subtile
// sub; the two buffers are distinct objects so the compiler need not order
// the loads against the reads of the other buffer); register-staged engines
// prefetch into registers and use one buffer.
// start() runs once the first subtile's loads are queued (work whose own
// loads should overlap them: the query rows, the merge's partials).
template <class E, int NT, bool TAIL, class S, class F>
__device__ __forceinline__ void stream_subtiles_t(char* bufA, char* bufB, const typename E::T* kp,
                                                  const typename E::T* vp, int nsub, int last_rows, int D, int tid,
                                                  S&& start, F&& compute) {
  // Without a partial last subtile (TAIL false) every subtile holds 64 rows
  // and the loop carries no tail logic.
  auto rows_of = [&](int sub) { return (TAIL && sub == nsub - 1) ? last_rows : kSub; };
  if constexpr (E::kDMA) {
    // Direct loads from wave-uniform bases with per-lane offsets computed
    // once (no per-load address arithmetic).
    typename E::template LoadOffsets<NT> lo;
    E::template load_offsets<NT>(lo, tid);
    auto issue = [&](int sub, char* buf) {
      if (TAIL) {
        load_subtile<E, NT, false>(kp + sub * (int64_t)kSub * D, lo, buf, tid, rows_of(sub));
        load_subtile<E, NT, true>(vp + sub * (int64_t)kSub * D, lo, buf + E::TB, tid, rows_of(sub));
      } else {
        E::template begin_uniform<NT, false>(kp + sub * (int64_t)kSub * D, lo, buf, tid);
        E::template begin_uniform<NT, true>(vp + sub * (int64_t)kSub * D, lo, buf + E::TB, tid);
      }
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
  } else {
    typename E::template Stage<NT> st;
    E::template begin<NT>(st, kp, vp, bufA, tid, rows_of(0));
    start();
    E::template land<NT>(st, bufA, tid);
    // Also tell the compiler that every vector-memory load issued so far
    // (the query fragments) has completed, so that it emits no vmcnt waits
    // inside the loop, where the only outstanding loads are the next
    // subtile's.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    const int64_t step_elems = (int64_t)kSub * D;
    for (int sub = 0; sub < nsub; ++sub) {
      const bool more = sub + 1 < nsub;
      if (more)
        E::template begin<NT>(st, kp + (sub + 1) * step_elems, vp + (sub + 1) * step_elems, bufA, tid,
                              rows_of(sub + 1));
      compute(bufA, sub);
      if (more) {
        __syncthreads();
        E::template land<NT>(st, bufA, tid);
      }
      __syncthreads();
    }
  }
}

// stream_subtiles_t, its tail handling compiled in only where the last
// subtile is partial (last_rows < 64).
template <class E, int NT, class S, class F>
__device__ __forceinline__ void stream_subtiles(char* bufA, char* bufB, const typename E::T* kp,
                                                const typename E::T* vp, int nsub, int last_rows, int D, int tid,
                                                S&& start, F&& compute) {
  if (last_rows < kSub) stream_subtiles_t<E, NT, true>(bufA, bufB, kp, vp, nsub, last_rows, D, tid, start, compute);
  else stream_subtiles_t<E, NT, false>(bufA, bufB, kp, vp, nsub, last_rows, D, tid, start, compute);
}

// K-ahead stream for direct-load engines (gather; no causal mask, only the
// padding rows of a partial last subtile are masked):
// each buffer holds a K subtile then a V subtile (TB bytes each). Step sub
// loads K of sub+2 and V of sub+1, computes the scores of sub+1 while the
// weights and P.V of sub run, and ends at the barrier that publishes the
// loads. Buffer use: K(sub) in buf[sub % 2], V(sub) in buf[sub % 2] + TB;
// K(sub+2) overwrites K(sub), read in the step before (or the prologue,
// followed by its own barrier), V(sub+1) overwrites V(sub-1), read in the
// step before.
template <class E, int NT, bool ON, bool TAIL, class S>
__device__ __forceinline__ void stream_k_ahead_t(E& eng, char* bufA, char* bufB, const typename E::T* kp,
                                                 const typename E::T* vp, int nsub, int last_rows, int tid, int lane,
                                                 float sl2, S&& start) {
  constexpr int64_t SE = (int64_t)kSub * E::kD;
  const int h = lane >> 5;
  constexpr bool tail = TAIL;  // the last subtile is partial: clamped loads, masked scores
  auto rows_of = [&](int sub) { return (TAIL && sub == nsub - 1) ? last_rows : kSub; };
  typename E::template LoadOffsets<NT> lo;
  E::template load_offsets<NT>(lo, tid);
  // Loads of subtile sub (K: IS_V false); only a TAIL stream can meet a partial one.
  auto ld = [&](auto is_v, const typename E::T* p, int sub, char* buf) {
    constexpr bool V = decltype(is_v)::value;
    if (TAIL) load_subtile<E, NT, V>(p, lo, buf, tid, rows_of(sub));
    else E::template begin_uniform<NT, V>(p, lo, buf, tid);
  };
  using KL = std::integral_constant<bool, false>;
  using VL = std::integral_constant<bool, true>;
  ld(KL{}, kp, 0, bufA);
  ld(VL{}, vp, 0, bufA + E::TB);
  if (nsub > 1) ld(KL{}, kp + SE, 1, bufB);
  start();  // e.g. the query rows, under the first K/V loads
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): see stream_subtiles
  lds_dma_wait();
  __syncthreads();
  f32x16 sa[2], sb[2];
  float ma = kNegInf, mb = kNegInf;
  if (ON) {
    eng.qk(bufA, lane, sa);
    if (tail && nsub == 1) mask_rows(sa, last_rows, h);
    ma = E::rowmax(sa, sl2);
  }
  __syncthreads();
  // A step with a next subtile (its scores are computed here). Both loads
  // it queues are read by the very next step (K(sub+2) for that step's
  // scores, V(sub+1) for its P.V), so the step ends waiting for all of this
  // wave's loads before the barrier that publishes them to the other waves.
  auto full = [&](int sub, char* bc, char* bn, f32x16(&sc)[2], f32x16(&sn)[2], float mc, float& mn) {
    const bool k2 = sub + 2 < nsub;
    ld(VL{}, vp + (sub + 1) * SE, sub + 1, bn + E::TB);
    if (k2) ld(KL{}, kp + (sub + 2) * SE, sub + 2, bc);
    if (ON) {
      eng.rescale(mc);
      eng.fused(bn, sn, sc, bc + E::TB, lane, sl2, mn);
      if (tail && sub + 1 == nsub - 1) {
        mask_rows(sn, last_rows, h);
        mn = E::rowmax(sn, sl2);
      }
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
                                               const typename E::T* vp, int nsub, int last_rows, int tid, int lane,
                                               bool on, float sl2, S&& start) {
  if (last_rows < kSub) {
    if (on) stream_k_ahead_t<E, NT, true, true>(eng, bufA, bufB, kp, vp, nsub, last_rows, tid, lane, sl2, start);
    else stream_k_ahead_t<E, NT, false, true>(eng, bufA, bufB, kp, vp, nsub, last_rows, tid, lane, sl2, start);
  } else {
    if (on) stream_k_ahead_t<E, NT, true, false>(eng, bufA, bufB, kp, vp, nsub, last_rows, tid, lane, sl2, start);
    else stream_k_ahead_t<E, NT, false, false>(eng, bufA, bufB, kp, vp, nsub, last_rows, tid, lane, sl2, start);
  }
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
}  // namespace moba
