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
// Mapping on gfx950: a wave owns 32 consecutive queries (they share c).
// Scores come from bf16 MFMA 32x32x16 with the block means as the A operand
// (rows = blocks) and the queries as the B operand (columns = queries), so
// lane l holds 16 block scores of query l%32 and the per-query top-k runs in
// registers; the two lane halves merge their lists with one exchange.
// The means enter as a bf16 hi/lo pair (two MFMA passes, fp32 accumulate);
// fp32 inputs use fp32 MFMA on the fp32 means.
//
// Exactness: every fast score carries a rounding bound
//   eps = gamma * ||q_t||_2 * max_j ||kbar_j||_2   (Cauchy-Schwarz),
// gamma covering the hi/lo residual and the fp32 accumulation. If the gap
// between the last kept and the first dropped fast score is not above
// 2*eps, the query's tracked candidates (or, if the bound reaches beyond the
// tracked list, all its eligible blocks) are re-scored in fp64 from the fp64
// means and selected again. The selection then equals the one made with
// exact scores, except for scores equal to within fp64 rounding.
//
// Outputs: block_idx row (ascending, own block included, -1 padded), and for
// each kept past block an atomic increment of that block's query count whose
// return value is the query's position in the block's list (rank).
#include "common.h"
#include "launch.h"

namespace moba {

namespace {

constexpr int kNoBlock = 0x7fffffff;

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

// Query fragment held by one lane: the lane's half of q_t's coordinates.
template <typename T, int D>
struct QFrag;

template <int D>
struct QFrag<bf16, D> {
  static constexpr int KC = D / 16;
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
  // fp64 dot of this lane's coordinates with row kb (fp64), in a fixed order.
  __device__ double dot64(const double* kb, int h) const {
    double s = 0.0;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) s = __builtin_fma((double)(float)f[kk][e], kb[16 * kk + 8 * h + e], s);
    return s;
  }
  __device__ f32x16 scores(const bf16* hi, const bf16* lo, int h) const {
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(hi + 16 * kk + 8 * h);
      acc = mfma_bf16(a, f[kk], acc);
    }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lo + 16 * kk + 8 * h);
      acc = mfma_bf16(a, f[kk], acc);
    }
    return acc;
  }
  // Relative rounding bound of a fast score: hi/lo residual (<= 2^-16 of
  // each mean coordinate, taken as 2^-15) plus 2D+16 fp32 accumulation
  // steps at 2^-22 each (a 4x margin over rounding to nearest).
  static __device__ constexpr float gamma() { return 3.0517578e-05f + (2 * D + 16) * 2.3841858e-07f; }
};

template <int D>
struct QFrag<float, D> {
  static constexpr int KC = D / 2;
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
  __device__ double dot64(const double* kb, int h) const {
    double s = 0.0;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) s = __builtin_fma((double)f[kk], kb[2 * kk + h], s);
    return s;
  }
  __device__ f32x16 scores(const float* k32, int h) const {
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) acc = mfma_f32(k32[2 * kk + h], f[kk], acc);
    return acc;
  }
  // fp32 products and 2D+16 accumulation steps at 2^-22 each.
  static __device__ constexpr float gamma() { return (2 * D + 16) * 2.3841858e-07f; }
};

}  // namespace

template <typename T, int D, int TT>
__global__ __launch_bounds__(256) void gate_topk_kernel(GateArgs a) {
  const int lane = threadIdx.x & 63, h = lane >> 5, col = lane & 31;
  const int64_t groups_per_head = a.seq_len / 32;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= a.bh * groups_per_head) return;  // no barriers in this kernel
  const int64_t bh = g / groups_per_head;
  const int64_t t0 = (g % groups_per_head) * 32;
  const int64_t t = t0 + col;
  const int c = (int)(t0 / a.block_size);
  const int NB = (int)a.n_blocks;
  const int n_elig = a.causal ? c : NB - 1;
  const int m = min(a.k_eff - 1, n_elig);
  const int slots = a.k_eff - 1;
  int32_t* idx_row = a.block_idx + (bh * a.seq_len + t) * a.top_k;
  int32_t* rank_row = a.rank + (bh * a.seq_len + t) * (int64_t)slots;
  int32_t* cnt = a.count + bh * NB;

  if (m == 0 || m == n_elig) {
    // Only the own block (top_k = 1), or every eligible block is kept
    // (early blocks, or top_k >= n_blocks): no scores are needed.
    if (h == 0) {
      int col_out = 0, slot = 0;
      if (m == 0) {
        idx_row[col_out++] = c;
      } else {
        const int jend = a.causal ? c + 1 : NB;
        for (int j = 0; j < jend; ++j) {
          idx_row[col_out++] = j;
          if (j != c) rank_row[slot++] = atomicAdd(cnt + j, 1);
        }
      }
      for (; col_out < a.top_k; ++col_out) idx_row[col_out] = -1;
    }
    return;
  }

  // ---- fast scores over all eligible blocks, top-TT per lane half
  QFrag<T, D> qf;
  const T* qrow = reinterpret_cast<const T*>(a.q) + (bh * a.seq_len + t) * D;
  qf.load(qrow, h);
  float qss = qf.sumsq();
  qss += shfl_xor32(qss);
  const float qnorm = __builtin_sqrtf(qss) * 1.0001f;

  float ls[TT];
  int lj[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    ls[i] = kNegInf;
    lj[i] = kNoBlock;
  }
  const int jend = a.causal ? c : NB;
  for (int jt = 0; jt < jend; jt += 32) {
    const int arow = min(jt + col, NB - 1);
    f32x16 acc;
    if constexpr (sizeof(T) == 2) {
      acc = qf.scores(a.kbar_hi + (bh * NB + arow) * D, a.kbar_lo + (bh * NB + arow) * D, h);
    } else {
      acc = qf.scores(a.kbar32 + (bh * NB + arow) * D, h);
    }
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
  // Merge the two lane halves (each lane merges the other's list into its
  // own; the order is strict, so both halves end with the same list).
  {
    float ps[TT];
    int pj[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      ps[i] = shfl_xor32(ls[i]);
      pj[i] = shfl_xor32(lj[i]);
    }
#pragma unroll
    for (int i = 0; i < TT; ++i) insert_full(ls, lj, ps[i], pj[i]);
  }

  // ---- exactness check and fp64 re-scoring where the cut is uncertain
  const float eps = QFrag<T, D>::gamma() * qnorm * a.norm[bh] + 1e-30f;
  const float gap = ls[m - 1] - ls[m];
  int sel[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) sel[i] = lj[i];
  if (!(gap > 2.f * eps)) {
    const double* kb64 = a.kbar64 + bh * NB * (int64_t)D;
    const bool tracked = n_elig <= TT || ls[TT - 1] < ls[m - 1] - 2.f * eps;
    double es[TT];
    int ej[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      es[i] = -__builtin_huge_val();
      ej[i] = kNoBlock;
    }
    if (tracked) {
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        if (lj[i] != kNoBlock) {
          double p = qf.dot64(kb64 + (int64_t)lj[i] * D, h);
          p += shfl_xor32(p);
          insert_full64(es, ej, p, lj[i]);
        }
      }
    } else {
      for (int j = 0; j < jend; ++j) {
        if (j == c) continue;
        double p = qf.dot64(kb64 + (int64_t)j * D, h);
        p += shfl_xor32(p);
        if (better64(p, j, es[TT - 1], ej[TT - 1])) insert_full64(es, ej, p, j);
      }
    }
#pragma unroll
    for (int i = 0; i < TT; ++i) sel[i] = ej[i];
  }

  // ---- write the row: kept past blocks ascending with the own block
  if (h == 0) {
    // sort the first m entries by block index (m <= TT - 2)
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
        rank_row[i] = atomicAdd(cnt + j, 1);
      }
    }
    if (!own_done) idx_row[col_out++] = c;
    for (; col_out < a.top_k; ++col_out) idx_row[col_out] = -1;
  }
}

template <typename T, int D>
static hipError_t gate_launch_t(const GateArgs& a, hipStream_t s) {
  const int64_t groups = a.bh * (a.seq_len / 32);
  const dim3 grid((unsigned)((groups + 3) / 4));
  const int m = a.k_eff - 1;
  KernelTimer timer(s, "gate_topk");
  if (m <= 2)
    hipLaunchKernelGGL((gate_topk_kernel<T, D, 4>), grid, dim3(256), 0, s, a);
  else if (m <= 6)
    hipLaunchKernelGGL((gate_topk_kernel<T, D, 8>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gate_topk_kernel<T, D, kMaxSlots + 2>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gate(const GateArgs& a, hipStream_t s) {
  if (a.bf16_in) return a.head_dim == 128 ? gate_launch_t<bf16, 128>(a, s) : gate_launch_t<bf16, 64>(a, s);
  return a.head_dim == 128 ? gate_launch_t<float, 128>(a, s) : gate_launch_t<float, 64>(a, s);
}

}  // namespace moba
