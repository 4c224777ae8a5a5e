// Gate scores, future-block mask and top-k block selection (one kernel).
//
// Method («月之暗面 MoBA 论文解读» §3.1 and §4.1; the hncyxsy.com MOBA
// article §3; «MoBA 复现代码跑不通…» §3.2):
//  * each query t in block c scores every eligible block j by q_t . kbar_j,
//    where kbar_j is the block's mean key; with causal routing only j < c is
//    eligible (future blocks are masked), otherwise every j != c;
//  * the own block c is never scored: it is always kept (its mean contains
//    keys after t);
//  * the other min(top_k, n_blocks) - 1 slots go to the best eligible
//    scores, equal scores resolved towards the lower block index.
//
// Mapping on gfx950: a workgroup owns 128 consecutive queries of one head,
// a wave 32 of them (they share c because block_size is a multiple of 64).
// Tiles of 32 pooled keys are staged in LDS once per workgroup. Scores come
// from bf16 MFMA 32x32x16 with the pooled keys as the A operand (rows =
// blocks) and the queries as the B operand (columns = queries), so lane l
// holds 16 block scores of query l%32 and the per-query top-k runs in
// registers; the two lane halves merge their lists with one exchange. The
// pooled keys enter as a bf16 hi/lo pair (two MFMA passes, fp32 accumulate);
// fp32 inputs use fp32 MFMA on the fp32 means.
//
// Exactness: every fast score carries a rounding bound
//   eps = gamma * ||q_t||_2 * max_j ||kbar_j||_2   (Cauchy-Schwarz),
// gamma covering the hi/lo residual and the fp32 accumulation. If the gap
// between the last kept and the first dropped fast score is not above
// 2*eps, the query's tracked candidates (or, if the bound reaches beyond the
// tracked list, all its eligible blocks) are re-scored in fp64 from the fp64
// means and selected again; the wave does this together, one such query at
// a time, 64 lanes sharing the dot products. The selection then equals the
// one made with exact scores, except for scores equal to within fp64
// rounding.
//
// Output: the block_idx row (ascending, own block included, -1 padded).
// A second kernel (rank_kernel) then numbers each query inside the lists
// of the past blocks it kept: an LDS histogram per 1024 queries plus one
// global atomic per (workgroup, block), so hot blocks see few atomics.
#include "common.h"
#include "launch.h"

namespace moba {

namespace {

constexpr int kNoBlock = 0x7fffffff;
constexpr int kGateQ = 128;         // queries per workgroup
constexpr int kTileB = 32;          // pooled keys per LDS tile
constexpr int kLdsBinsMax = 8192;   // per-workgroup histogram bins kept in LDS
constexpr int kRankQ = 1024;        // queries per rank workgroup

// Strict order: higher score first, then lower block index.
__device__ __forceinline__ bool better(float s1, int j1, float s2, int j2) {
  return s1 > s2 || (s1 == s2 && j1 < j2);
}
__device__ __forceinline__ bool better64(double s1, int j1, double s2, int j2) {
  return s1 > s2 || (s1 == s2 && j1 < j2);
}

// Insert (s, j) into a list sorted by `better`, keeping its length.
template <int N>
__device__ __forceinline__ void insert_full(float (&ls)[N], int (&lj)[N], float s, int j) {
#pragma unroll
  for (int i = N - 1; i >= 0; --i) {
    const bool here = better(s, j, ls[i], lj[i]);
    const bool above = (i > 0) ? better(s, j, ls[i - 1], lj[i - 1]) : false;
    const float ns = above ? ls[i - 1] : (here ? s : ls[i]);
    const int nj = above ? lj[i - 1] : (here ? j : lj[i]);
    ls[i] = ns;
    lj[i] = nj;
  }
}
template <int N>
__device__ __forceinline__ void insert_full64(double (&ls)[N], int (&lj)[N], double s, int j) {
#pragma unroll
  for (int i = N - 1; i >= 0; --i) {
    const bool here = better64(s, j, ls[i], lj[i]);
    const bool above = (i > 0) ? better64(s, j, ls[i - 1], lj[i - 1]) : false;
    const double ns = above ? ls[i - 1] : (here ? s : ls[i]);
    const int nj = above ? lj[i - 1] : (here ? j : lj[i]);
    ls[i] = ns;
    lj[i] = nj;
  }
}

// Per-dtype query fragment (the lane's half of q_t's coordinates), pooled
// key tile layout in LDS, and the fast-score rounding bound.
template <typename T, int D>
struct GateOps;

template <int D>
struct GateOps<bf16, D> {
  static constexpr int KC = D / 16;
  static constexpr int KR = D + 8;  // LDS row stride (elements), 16-byte aligned rows
  static constexpr int TILE_BYTES = 2 * kTileB * KR * 2;
  bf16x8 f[KC];
  __device__ void load(const bf16* qrow, int h) {
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) f[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk + 8 * h);
  }
  __device__ float sumsq() const {
    float s = 0.f;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)f[kk][e];
        s = __builtin_fmaf(x, x, s);
      }
    return s;
  }
  // Stage rows j0 .. j0+31 (clamped to the last block) of hi and lo.
  static __device__ void stage(char* lds, const GateArgs& a, int64_t bh, int j0, int tid) {
    bf16* hi = reinterpret_cast<bf16*>(lds);
    bf16* lo = hi + kTileB * KR;
    constexpr int CH = kTileB * D / 8;  // 16-byte chunks per tile (per hi or lo)
#pragma unroll
    for (int i = tid; i < 2 * CH; i += 256) {
      const int which = i / CH, id = i % CH;
      const int row = id / (D / 8), cc = id % (D / 8);
      const int j = min(j0 + row, (int)a.n_blocks - 1);
      const bf16* src = (which ? a.kbar_lo : a.kbar_hi) + (bh * a.n_blocks + j) * D + 8 * cc;
      *reinterpret_cast<u32x4*>((which ? lo : hi) + row * KR + 8 * cc) = *reinterpret_cast<const u32x4*>(src);
    }
  }
  __device__ f32x16 scores(const char* lds, int col, int h) const {
    const bf16* hi = reinterpret_cast<const bf16*>(lds) + col * KR + 8 * h;
    const bf16* lo = hi + kTileB * KR;
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(hi + 16 * kk), f[kk], acc);
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(lo + 16 * kk), f[kk], acc);
    return acc;
  }
  // Relative rounding bound of a fast score: hi/lo residual (<= 2^-16 of
  // each mean coordinate, taken as 2^-15) plus 2D+16 fp32 accumulation
  // steps at 2^-22 each (a 4x margin over rounding to nearest).
  static __device__ constexpr float gamma() { return 3.0517578e-05f + (2 * D + 16) * 2.3841858e-07f; }
};

template <int D>
struct GateOps<float, D> {
  static constexpr int KC = D / 2;
  static constexpr int KR = D + 2;  // LDS row stride (floats): conflict-free column reads
  static constexpr int TILE_BYTES = kTileB * KR * 4;
  float f[KC];
  __device__ void load(const float* qrow, int h) {
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) f[kk] = qrow[2 * kk + h];
  }
  __device__ float sumsq() const {
    float s = 0.f;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) s = __builtin_fmaf(f[kk], f[kk], s);
    return s;
  }
  static __device__ void stage(char* lds, const GateArgs& a, int64_t bh, int j0, int tid) {
    float* kt = reinterpret_cast<float*>(lds);
    constexpr int CH = kTileB * D / 2;  // 8-byte chunks per tile
    for (int id = tid; id < CH; id += 256) {
      const int row = id / (D / 2), cc = id % (D / 2);
      const int j = min(j0 + row, (int)a.n_blocks - 1);
      *reinterpret_cast<float2*>(kt + row * KR + 2 * cc) =
          *reinterpret_cast<const float2*>(a.kbar32 + (bh * a.n_blocks + j) * D + 2 * cc);
    }
  }
  __device__ f32x16 scores(const char* lds, int col, int h) const {
    const float* kt = reinterpret_cast<const float*>(lds) + col * KR + h;
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) acc = mfma_f32(kt[2 * kk], f[kk], acc);
    return acc;
  }
  // fp32 products and 2D+16 accumulation steps at 2^-22 each.
  static __device__ constexpr float gamma() { return (2 * D + 16) * 2.3841858e-07f; }
};

}  // namespace

template <typename T, int D, int TT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TT <= 4 ? 3 : 2))) void gate_topk_kernel(
    GateArgs a) {
  using Ops = GateOps<T, D>;
  extern __shared__ __align__(16) char smem[];
  char* tile = smem;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  const int64_t wg_per_head = (a.seq_len + kGateQ - 1) / kGateQ;
  const int64_t bh = blockIdx.x / wg_per_head;
  const int64_t qb = (blockIdx.x % wg_per_head) * kGateQ;
  const int64_t t0 = qb + 32 * w;
  const bool wave_on = t0 < a.seq_len;  // workgroup-uniform control flow below
  const int64_t t = wave_on ? t0 + col : qb;
  const int NB = (int)a.n_blocks;
  const int c = (int)(t / a.block_size);
  const int n_elig = a.causal ? c : NB - 1;
  const int m = min(a.k_eff - 1, n_elig);
  const bool scoring = wave_on && m > 0 && m < n_elig;  // wave-uniform
  int32_t* idx_row = a.block_idx + (bh * a.seq_len + t) * a.top_k;

  // ---- fast scores over the eligible blocks, top-TT per lane half
  Ops qf;
  const T* qrow = reinterpret_cast<const T*>(a.q) + (bh * a.seq_len + t) * D;
  float qnorm = 0.f;
  if (scoring) {
    qf.load(qrow, h);
    float qss = qf.sumsq();
    qss += shfl_xor32(qss);
    qnorm = __builtin_sqrtf(qss) * 1.0001f;
  }
  float ls[TT];
  int lj[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    ls[i] = kNegInf;
    lj[i] = kNoBlock;
  }
  const int jend = a.causal ? c : NB;  // this wave's scan bound
  // Scan bound of the whole workgroup (its last valid query has the largest c).
  const int64_t t_last = min<int64_t>(qb + kGateQ, a.seq_len) - 1;
  const int wg_jend = a.causal ? (int)(t_last / a.block_size) : NB;
  for (int jt = 0; jt < wg_jend; jt += kTileB) {
    __syncthreads();
    Ops::stage(tile, a, bh, jt, tid);
    __syncthreads();
    if (!scoring || jt >= jend) continue;
    const f32x16 acc = qf.scores(tile, col, h);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = jt + crow(r, h);
      const bool ok = j < jend && j != c;
      const float s = ok ? acc[r] : kNegInf;
      // Blocks reach a lane in increasing j, so a strict test keeps the
      // lower index first among equal scores.
      if (s > ls[TT - 1]) {
#pragma unroll
        for (int i = TT - 1; i >= 0; --i) {
          const bool here = s > ls[i];
          const bool above = (i > 0) ? (s > ls[i - 1]) : false;
          const float ns = above ? ls[i - 1] : (here ? s : ls[i]);
          const int nj = above ? lj[i - 1] : (here ? j : lj[i]);
          ls[i] = ns;
          lj[i] = nj;
        }
      }
    }
  }

  int sel[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) sel[i] = lj[i];
  if (scoring) {
    // Merge the two lane halves (each lane merges the other's list into its
    // own; the order is strict, so both halves end with the same list).
    float ps[TT];
    int pj[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      ps[i] = shfl_xor32(ls[i]);
      pj[i] = shfl_xor32(lj[i]);
    }
#pragma unroll
    for (int i = 0; i < TT; ++i) insert_full(ls, lj, ps[i], pj[i]);
#pragma unroll
    for (int i = 0; i < TT; ++i) sel[i] = lj[i];

    // ---- exactness check: is the cut between kept and dropped blocks
    // farther apart than twice the fast scores' rounding bound?
    const float eps = Ops::gamma() * qnorm * a.norm[bh] + 1e-30f;
    const bool amb = !(ls[m - 1] - ls[m] > 2.f * eps);
    const bool tracked = n_elig <= TT || ls[TT - 1] < ls[m - 1] - 2.f * eps;
    // ---- fp64 re-scoring, one ambiguous query at a time, by the whole wave
    // (c, m and the eligible set are the same for every query of the wave).
    uint64_t pend = __builtin_amdgcn_ballot_w64(amb && h == 0);
    const double* kb64 = a.kbar64 + bh * NB * (int64_t)D;
    constexpr int SL = D / 8;    // 8-coordinate slices per candidate
    constexpr int G = 64 / SL;   // candidates per pass
    const int gi = lane / SL, sl = lane % SL;
    while (pend) {
      const int L = __builtin_ctzll(pend);
      pend &= pend - 1;
      const bool trk = __builtin_amdgcn_readlane((int)tracked, L);
      // This lane's slice of the ambiguous query's coordinates, in fp64.
      const T* qL = reinterpret_cast<const T*>(a.q) + (bh * a.seq_len + t0 + L) * D + 8 * sl;
      double qd[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) qd[e] = (double)(float)qL[e];
      int cj[TT];
#pragma unroll
      for (int i = 0; i < TT; ++i) cj[i] = __builtin_amdgcn_readlane(lj[i], L);
      double es[TT];
      int ej[TT];
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        es[i] = -__builtin_huge_val();
        ej[i] = kNoBlock;
      }
      // Candidates: the tracked list, or every eligible block when the
      // rounding band reaches past the list.
      const int ncand = trk ? TT : jend;
      for (int base = 0; base < ncand; base += G) {
        const int ci = base + gi;
        int j = kNoBlock;
        if (trk) {
#pragma unroll
          for (int i = 0; i < TT; ++i)
            if (ci == i) j = cj[i];
        } else if (ci < jend && ci != c) {
          j = ci;
        }
        double p = 0.0;
        if (j != kNoBlock) {
          const double* kr = kb64 + (int64_t)j * D + 8 * sl;
#pragma unroll
          for (int e = 0; e < 8; ++e) p = __builtin_fma(qd[e], kr[e], p);
        }
        // Sum the SL slices of each candidate (fixed order: deterministic).
#pragma unroll
        for (int w = SL / 2; w > 0; w >>= 1) p += __shfl_xor(p, w);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int jg = __builtin_amdgcn_readlane(j, g * SL);
          if (jg == kNoBlock) continue;
          const int lo_bits = __builtin_amdgcn_readlane((int)(__double_as_longlong(p) & 0xffffffff), g * SL);
          const int hi_bits = __builtin_amdgcn_readlane((int)(__double_as_longlong(p) >> 32), g * SL);
          const double pg = __longlong_as_double(((long long)hi_bits << 32) | (unsigned)lo_bits);
          if (better64(pg, jg, es[TT - 1], ej[TT - 1])) insert_full64(es, ej, pg, jg);
        }
      }
      if (col == L) {
#pragma unroll
        for (int i = 0; i < TT; ++i) sel[i] = ej[i];
      }
    }
  }

  // ---- write the row: kept past blocks ascending, with the own block
  if (!wave_on || h != 0) return;
  if (!scoring) {
    // Only the own block (m = 0), or every eligible block is kept.
    int col_out = 0;
    if (m == 0) {
      idx_row[col_out++] = c;
    } else {
      const int jstop = a.causal ? c + 1 : NB;
      for (int j = 0; j < jstop; ++j) idx_row[col_out++] = j;
    }
    for (; col_out < a.top_k; ++col_out) idx_row[col_out] = -1;
    return;
  }
  int srt[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) srt[i] = (i < m) ? sel[i] : kNoBlock;
#pragma unroll
  for (int i = 1; i < TT; ++i)
#pragma unroll
    for (int k = i; k > 0; --k) {
      const int x = srt[k - 1], y = srt[k];
      srt[k - 1] = min(x, y);
      srt[k] = max(x, y);
    }
  int col_out = 0;
  bool own_done = false;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    if (i < m) {
      const int j = srt[i];
      if (!own_done && c < j) {
        idx_row[col_out++] = c;
        own_done = true;
      }
      idx_row[col_out++] = j;
    }
  }
  if (!own_done) idx_row[col_out++] = c;
  for (; col_out < a.top_k; ++col_out) idx_row[col_out] = -1;
}

// Numbers every (query, kept past block) pair inside that block's query
// list: rank[q][slot] = position of q in the list of the slot's block.
// Workgroups of 1024 queries count their picks per block in LDS, reserve
// one contiguous range per block with a single global atomic, and add the
// range start to each pick's local position.
__global__ __launch_bounds__(256) void rank_kernel(GateArgs a) {
  extern __shared__ __align__(16) char smem[];
  int* bins = reinterpret_cast<int*>(smem);
  const int NB = (int)a.n_blocks;
  const bool lds_bins = NB <= kLdsBinsMax;
  const int64_t wg_per_head = (a.seq_len + kRankQ - 1) / kRankQ;
  const int64_t bh = blockIdx.x / wg_per_head;
  const int64_t q0 = (blockIdx.x % wg_per_head) * kRankQ;
  const int slots = a.k_eff - 1;
  int32_t* cnt = a.count + bh * NB;
  if (lds_bins)
    for (int i = threadIdx.x; i < NB; i += 256) bins[i] = 0;
  __syncthreads();
  for (int qq = threadIdx.x; qq < kRankQ; qq += 256) {
    const int64_t t = q0 + qq;
    if (t >= a.seq_len) break;
    const int c = (int)(t / a.block_size);
    const int32_t* row = a.block_idx + (bh * a.seq_len + t) * a.top_k;
    int32_t* rk = a.rank + (bh * a.seq_len + t) * (int64_t)slots;
    int s = 0;
    for (int i = 0; i < a.top_k; ++i) {
      const int j = row[i];
      if (j < 0) break;
      if (j == c) continue;
      rk[s++] = lds_bins ? atomicAdd(bins + j, 1) : atomicAdd(cnt + j, 1);
    }
  }
  if (!lds_bins) return;  // ranks are already global
  __syncthreads();
  for (int i = threadIdx.x; i < NB; i += 256) {
    const int n = bins[i];
    if (n) bins[i] = atomicAdd(cnt + i, n);
  }
  __syncthreads();
  for (int qq = threadIdx.x; qq < kRankQ; qq += 256) {
    const int64_t t = q0 + qq;
    if (t >= a.seq_len) break;
    const int c = (int)(t / a.block_size);
    const int32_t* row = a.block_idx + (bh * a.seq_len + t) * a.top_k;
    int32_t* rk = a.rank + (bh * a.seq_len + t) * (int64_t)slots;
    int s = 0;
    for (int i = 0; i < a.top_k; ++i) {
      const int j = row[i];
      if (j < 0) break;
      if (j == c) continue;
      rk[s++] += bins[j];
    }
  }
}

template <typename T, int D, int TT>
static void gate_go(const GateArgs& a, hipStream_t s, dim3 grid, int lds) {
  hipLaunchKernelGGL((gate_topk_kernel<T, D, TT>), grid, dim3(256), lds, s, a);
}

template <typename T, int D>
static hipError_t gate_launch_t(const GateArgs& a, hipStream_t s) {
  const int64_t wg_per_head = (a.seq_len + kGateQ - 1) / kGateQ;
  const dim3 grid((unsigned)(a.bh * wg_per_head));
  const int m = a.k_eff - 1;
  const int lds = GateOps<T, D>::TILE_BYTES;
  {
    KernelTimer timer(s, "gate_topk");
    if (m <= 2) gate_go<T, D, 4>(a, s, grid, lds);
    else if (m <= 6) gate_go<T, D, 8>(a, s, grid, lds);
    else gate_go<T, D, kMaxSlots + 2>(a, s, grid, lds);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.k_eff < 2) return e;
  const int64_t rank_wgs = a.bh * ((a.seq_len + kRankQ - 1) / kRankQ);
  const int rank_lds = a.n_blocks <= kLdsBinsMax ? (int)a.n_blocks * 4 : 0;
  {
    KernelTimer timer(s, "rank");
    hipLaunchKernelGGL(rank_kernel, dim3((unsigned)rank_wgs), dim3(256), rank_lds, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gate(const GateArgs& a, hipStream_t s) {
  if (a.bf16_in) return a.head_dim == 128 ? gate_launch_t<bf16, 128>(a, s) : gate_launch_t<bf16, 64>(a, s);
  return a.head_dim == 128 ? gate_launch_t<float, 128>(a, s) : gate_launch_t<float, 64>(a, s);
}

}  // namespace moba
