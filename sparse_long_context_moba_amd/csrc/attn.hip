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
//                 of one block, attends the block's keys up to each query
//                 (causal), then merges the query's past partials with the
//                 log-sum-exp rule and writes o in the input dtype.
//  dense_attn   — plain full attention (causal or not) with the same engine,
//                 the baseline MoBA is measured against.
//
// Engine (one wave = 32 queries): S^T = K Q^T on MFMA 32x32x16 bf16 (K from
// LDS as the A operand, Q held in registers as the B operand), so lane l
// holds 32 scores of query l%32 per 64 keys and the row statistics need a
// single exchange with lane l^32. P stays in registers and feeds
// O^T = V^T P^T directly as the B operand; the A operand reads V^T from an
// LDS copy that is transposed while it is staged. fp32 inputs use
// MFMA 32x32x2 f32 with the same register layout and untransposed V.
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
template <int D>
struct EngBF16 {
  using T = bf16;
  static constexpr int KC = D / 16, DT = D / 32;
  static constexpr int KS = D + 8;     // K row stride in LDS (elements)
  static constexpr int VS = kSub + 4;  // V^T row stride in LDS (elements)
  static constexpr int KELEMS = kSub * KS;
  static constexpr int LDS_BYTES = (kSub * KS + D * VS) * 2;
  static constexpr int KCH = kSub * D / 8;  // 16-byte chunks of a K subtile
  static constexpr int VPT = 16 * (D / 8);  // 4-key x 8-dim patches of a V subtile

  bf16x8 qf[KC];
  f32x16 o[DT];
  float m, l;

  template <int NT>
  struct Stage {
    u32x4 k[(KCH + NT - 1) / NT];
    u32x4 v[4 * ((VPT + NT - 1) / NT)];  // four key rows per patch
  };

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

  template <int NT>
  static __device__ __forceinline__ void fetch(Stage<NT>& st, const bf16* kp, const bf16* vp, int tid) {
#pragma unroll
    for (int i = 0; i < (KCH + NT - 1) / NT; ++i) {
      const int id = tid + NT * i;
      if (KCH % NT == 0 || id < KCH) {
        const int row = id / (D / 8), cc = id % (D / 8);
        st.k[i] = *reinterpret_cast<const u32x4*>(kp + (int64_t)row * D + 8 * cc);
      }
    }
#pragma unroll
    for (int i = 0; i < (VPT + NT - 1) / NT; ++i) {
      const int id = tid + NT * i;
      if (VPT % NT == 0 || id < VPT) {
        const int kg = id / (D / 8), dg = id % (D / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st.v[4 * i + r] = *reinterpret_cast<const u32x4*>(vp + (int64_t)(4 * kg + r) * D + 8 * dg);
      }
    }
  }

  template <int NT>
  static __device__ __forceinline__ void store(const Stage<NT>& st, bf16* Ks, bf16* Vs, int tid) {
#pragma unroll
    for (int i = 0; i < (KCH + NT - 1) / NT; ++i) {
      const int id = tid + NT * i;
      if (KCH % NT == 0 || id < KCH) {
        const int row = id / (D / 8), cc = id % (D / 8);
        *reinterpret_cast<u32x4*>(Ks + row * KS + 8 * cc) = st.k[i];
      }
    }
#pragma unroll
    for (int i = 0; i < (VPT + NT - 1) / NT; ++i) {
      const int id = tid + NT * i;
      if (VPT % NT == 0 || id < VPT) {
        const int kg = id / (D / 8), dg = id % (D / 8);
        const u32x4 r0 = st.v[4 * i], r1 = st.v[4 * i + 1], r2 = st.v[4 * i + 2], r3 = st.v[4 * i + 3];
        bf16* vd = Vs + (8 * dg) * VS + 4 * kg;
        // Element e of the four key rows -> V^T row (8*dg + e), keys 4*kg..4*kg+3.
#define MOBA_VT_PUT(e, W)                                                                    \
  *reinterpret_cast<u32x2*>(vd + (e) * VS) =                                               \
      ((e) & 1) ? u32x2{(r0.W >> 16) | (r1.W & 0xffff0000u), (r2.W >> 16) | (r3.W & 0xffff0000u)} \
                : u32x2{(r0.W & 0xffffu) | (r1.W << 16), (r2.W & 0xffffu) | (r3.W << 16)};
        MOBA_VT_PUT(0, x)
        MOBA_VT_PUT(1, x)
        MOBA_VT_PUT(2, y)
        MOBA_VT_PUT(3, y)
        MOBA_VT_PUT(4, z)
        MOBA_VT_PUT(5, z)
        MOBA_VT_PUT(6, w)
        MOBA_VT_PUT(7, w)
#undef MOBA_VT_PUT
      }
    }
  }

  template <bool MASK>
  __device__ __forceinline__ void step(const bf16* Ks, const bf16* Vs, int col, int h, int key0, int qpos, float sl2) {
    f32x16 s[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      s[nt] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (32 * nt + col) * KS + 16 * kk + 8 * h);
        s[nt] = mfma_bf16(a, qf[kk], s[nt]);
      }
    }
    online_softmax<MASK>(s, m, l, o, h, key0, qpos, sl2);
    bf16x8 pb[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) pb[nt][r >> 3][r & 7] = to_bf16(s[nt][r]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const bf16* vp = Vs + (32 * dt + col) * VS + 32 * nt + 16 * g + 4 * h;
          const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vp);
          const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vp + 8);
          const bf16x8 av = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = mfma_bf16(av, pb[nt][g], o[dt]);
        }
    }
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
  static constexpr int KC = D / 2, DT = D / 32;
  static constexpr int KS = D + 2;  // K row stride (floats): conflict-free column reads
  static constexpr int VS = D + 8;  // V row stride (floats): the two lane halves hit disjoint banks
  static constexpr int KELEMS = kSub * KS;
  static constexpr int LDS_BYTES = (kSub * KS + kSub * VS) * 4;
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
  template <int NT>
  static __device__ __forceinline__ void fetch(Stage<NT>& st, const float* kp, const float* vp, int tid) {
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
  template <int NT>
  static __device__ __forceinline__ void store(const Stage<NT>& st, float* Ks, float* Vs, int tid) {
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
  __device__ __forceinline__ void step(const float* Ks, const float* Vs, int col, int h, int key0, int qpos, float sl2) {
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

}  // namespace

// ------------------------------------------------------- past-block gather
template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void gather_attn_kernel(AttnArgs a) {
  using E = typename EngOf<T, D>::type;
  constexpr int NT = 64 * NW, M = 32 * NW;
  extern __shared__ __align__(16) char smem[];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vs = Ks + E::KELEMS;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;

  // Tiles are numbered per (head, block) in order; consecutive tiles share a
  // block's K/V. Workgroups are dealt round-robin over the 8 XCDs, so give
  // each XCD one contiguous range of tiles to keep a block's K/V in one L2.
  const int64_t nblk = a.bh * a.n_blocks;
  const int total = a.tile_start[nblk];
  const int chunk = (total + 7) / 8;
  const int li = blockIdx.x / 8;
  if (li >= chunk) return;
  const int L = (int)(blockIdx.x % 8) * chunk + li;
  if (L >= total) return;
  int64_t lo = 0, hi = nblk;  // tile_start[lo] <= L < tile_start[hi]
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (a.tile_start[mid] <= L) lo = mid;
    else hi = mid;
  }
  const int64_t blk = lo;
  const int64_t bh = blk / a.n_blocks, j = blk % a.n_blocks;
  const int64_t e0 = a.offset[blk] + (int64_t)(L - a.tile_start[blk]) * M;
  const int64_t e1 = min<int64_t>(a.offset[blk + 1], e0 + M);
  const int64_t e = e0 + 32 * w + col;
  const bool valid = e < e1;
  const bool wave_on = e0 + 32 * w < e1;
  const int slots = a.k_eff - 1;
  const int ev = a.qlist[valid ? e : e0];
  const int t = ev / slots;

  E eng;
  eng.init();
  const T* q = reinterpret_cast<const T*>(a.q);
  if (wave_on) eng.load_q(q + (bh * a.seq_len + t) * D, h);
  const T* kp = reinterpret_cast<const T*>(a.k) + (bh * a.seq_len + j * a.block_size) * D;
  const T* vp = reinterpret_cast<const T*>(a.v) + (bh * a.seq_len + j * a.block_size) * D;
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int nsub = (int)(a.block_size / kSub);
  typename E::template Stage<NT> st;
  E::template fetch<NT>(st, kp, vp, tid);
  for (int sub = 0; sub < nsub; ++sub) {
    __syncthreads();
    E::template store<NT>(st, Ks, Vs, tid);
    __syncthreads();
    if (sub + 1 < nsub) E::template fetch<NT>(st, kp + (int64_t)(sub + 1) * kSub * D, vp + (int64_t)(sub + 1) * kSub * D, tid);
    if (wave_on) eng.template step<false>(Ks, Vs, col, h, 0, 0, sl2);
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
  extern __shared__ __align__(16) char smem[];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vs = Ks + E::KELEMS;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  // Heavier tiles (later in the sequence) first, heads interleaved.
  const int64_t ntile = a.seq_len / M;
  const int64_t tile = ntile - 1 - blockIdx.x / a.bh;
  const int64_t bh = blockIdx.x % a.bh;
  const int q0 = (int)(tile * M);
  const int c = (int)(q0 / a.block_size);
  const int kb = DENSE ? 0 : (int)(c * a.block_size);
  const int kend = a.causal ? q0 + M : (DENSE ? (int)a.seq_len : (int)(kb + a.block_size));
  const int qw0 = q0 + 32 * w;
  const int t = qw0 + col;

  E eng;
  eng.init();
  const T* q = reinterpret_cast<const T*>(a.q);
  eng.load_q(q + (bh * a.seq_len + t) * D, h);
  const T* kp = reinterpret_cast<const T*>(a.k) + (bh * a.seq_len + kb) * D;
  const T* vp = reinterpret_cast<const T*>(a.v) + (bh * a.seq_len + kb) * D;
  const float sl2 = kLog2e / __builtin_sqrtf((float)D);
  const int nsub = (kend - kb) / kSub;
  typename E::template Stage<NT> st;
  E::template fetch<NT>(st, kp, vp, tid);
  // Subtiles entirely before the workgroup's first query need no mask; with
  // causal attention the last M/64 subtiles hold the diagonal.
  const int nfree = a.causal ? (q0 - kb) / kSub : nsub;
  int sub = 0;
  for (; sub < nfree; ++sub) {
    __syncthreads();
    E::template store<NT>(st, Ks, Vs, tid);
    __syncthreads();
    if (sub + 1 < nsub) E::template fetch<NT>(st, kp + (int64_t)(sub + 1) * kSub * D, vp + (int64_t)(sub + 1) * kSub * D, tid);
    eng.template step<false>(Ks, Vs, col, h, 0, 0, sl2);
  }
  for (; sub < nsub; ++sub) {
    __syncthreads();
    E::template store<NT>(st, Ks, Vs, tid);
    __syncthreads();
    if (sub + 1 < nsub) E::template fetch<NT>(st, kp + (int64_t)(sub + 1) * kSub * D, vp + (int64_t)(sub + 1) * kSub * D, tid);
    const int key0 = kb + sub * kSub;
    // Skip a subtile whose keys all come after every query of this wave.
    if (key0 <= qw0 + 31) eng.template step<true>(Ks, Vs, col, h, key0, t, sl2);
  }

  const float lt = pair_sum(eng.l);
  if (DENSE) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int dt = 0; dt < E::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) eng.o[dt][r] *= inv;
  } else {
    // Merge with the past-block partials: one softmax over all chosen keys.
    const int n_elig = a.causal ? c : (int)a.n_blocks - 1;
    const int n = min(a.k_eff - 1, n_elig);
    const int slots = a.k_eff - 1;
    const int64_t rec0 = (bh * a.seq_len + t) * (int64_t)slots;
    const float lse_d = eng.m + fast_log2(lt);
    float mx = lse_d;
    for (int s = 0; s < n; ++s) mx = fmaxf(mx, a.part_lse[rec0 + s]);
    const float wd = fast_exp2(lse_d - mx);
    float wsum = wd;
    const float sd = wd / lt;
#pragma unroll
    for (int dt = 0; dt < E::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) eng.o[dt][r] *= sd;
    const T* po = reinterpret_cast<const T*>(a.part_o);
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
    const float inv = 1.f / wsum;
#pragma unroll
    for (int dt = 0; dt < E::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) eng.o[dt][r] *= inv;
  }
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
  hipError_t e = prep_lds(kern, E::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int64_t grid = (a.max_tiles + 7) / 8 * 8;
  KernelTimer timer(s, "gather_attn");
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NW), E::LDS_BYTES, s, a);
  return hipGetLastError();
}

template <typename T, int D, bool DENSE>
hipError_t diag_t(const AttnArgs& a, hipStream_t s) {
  using E = typename EngOf<T, D>::type;
  // 128-query tiles when they stay inside one block (and one sequence), else 64.
  const bool four = DENSE ? (a.seq_len % 128 == 0) : (a.block_size % 128 == 0);
  const char* name = DENSE ? "dense_attn" : "diag_merge";
  if (four) {
    auto kern = diag_attn_kernel<T, D, 4, DENSE>;
    hipError_t e = prep_lds(kern, E::LDS_BYTES);
    if (e != hipSuccess) return e;
    KernelTimer timer(s, name);
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.bh * (a.seq_len / 128))), dim3(256), E::LDS_BYTES, s, a);
  } else {
    auto kern = diag_attn_kernel<T, D, 2, DENSE>;
    hipError_t e = prep_lds(kern, E::LDS_BYTES);
    if (e != hipSuccess) return e;
    KernelTimer timer(s, name);
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.bh * (a.seq_len / 64))), dim3(128), E::LDS_BYTES, s, a);
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

}  // namespace moba
