// Block pooling of K: the gate's block summary.
//
// The gate of MoBA scores each block by the inner product of the query with
// the mean of the block's keys along the sequence («月之暗面 MoBA 论文解读»
// §3.1, gating.score_fn = mean_pool; the hncyxsy.com MOBA article §3). The
// article's §3 also names max pooling, and the two combined (read here as
// their sum), as options: the same pass computes any of the three.
//
// One pass, bound by HBM bandwidth: one workgroup per (head, block) reads
// the block's keys with 16-byte loads (several in flight per thread),
// accumulates in fp64 (and/or takes the running max) per thread, reduces
// across row groups in a fixed order, and writes the pooled key in fp64
// (exact re-scoring), fp32, and as a bf16 hi/lo pair (hi = bf16(x),
// lo = bf16(x - hi)) for the MFMA gate, plus the block's L2 norm (rounded
// up) for the gate's rounding bound. It also clears the block's query
// counts (one per query head reading this key/value head), which the gate's
// ranking fills. K is read exactly once; the fixed
// reduction order keeps results bit-stable.
#include "common.h"
#include "launch.h"

namespace moba {

// U rows per thread are loaded before they are accumulated (in row order);
// a block's last pass loads only the rows it holds (a block can hold any
// number of tokens from 1 to block_size).
// MODE selects the summary (moba_pooling_t): 0 mean, 1 max, 2 mean + max.
// The max is exact in any order (fp32 holds every input value).
template <typename T, int D, int U, int MODE>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int TPR = D / VEC;         // threads per row
  constexpr int RG = 256 / TPR;        // rows per pass
  constexpr bool SUM = MODE != 1, MAX = MODE != 0;
  __shared__ double red[SUM ? RG : 1][D];
  __shared__ float redm[MAX ? RG : 1][D];
  __shared__ double sq[D];
  const int tid = threadIdx.x;
  const int rg = tid / TPR, cv = tid % TPR;
  // Work item: one block of one key/value head of one sequence.
  const int64_t blk = blockIdx.x;  // the block's index in the pooled-key arrays
  const int64_t si = seq_find_u(a.sq, kSeqBlk, a.kv_heads, blk, a.block_size);
  const SeqAt sa = seq_at_u(a.sq, si, a.block_size);
  const int64_t r = blk - a.kv_heads * sa.blk0;
  const int64_t hk = r / sa.nb, j = r % sa.nb;
  // Rows of block j; the sequence's last block holds the remaining tokens.
  const int Bs = (int)min<int64_t>(a.block_size, sa.len - j * a.block_size);
  const T* base = reinterpret_cast<const T*>(a.k) + (sa.tok0 * a.kv_heads + hk * sa.len + j * a.block_size) * D +
                  cv * VEC;
  double acc[VEC];
  float mx[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    acc[e] = 0.0;
    mx[e] = -__builtin_inff();
  }
  auto take = [&](int e, float x) {
    if (SUM) acc[e] += (double)x;
    if (MAX) mx[e] = fmaxf(mx[e], x);
  };
  auto take_row = [&](const u32x4& raw) {
    if constexpr (sizeof(T) == 2) {
      const unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        take(2 * e, __uint_as_float(w[e] << 16));
        take(2 * e + 1, __uint_as_float(w[e] & 0xffff0000u));
      }
    } else {
      take(0, __uint_as_float(raw.x));
      take(1, __uint_as_float(raw.y));
      take(2, __uint_as_float(raw.z));
      take(3, __uint_as_float(raw.w));
    }
  };
  int r0 = rg;
  for (; r0 + (U - 1) * RG < Bs; r0 += U * RG) {
    u32x4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = *reinterpret_cast<const u32x4*>(base + (int64_t)(r0 + u * RG) * D);
#pragma unroll
    for (int u = 0; u < U; ++u) take_row(raw[u]);
  }
  for (; r0 < Bs; r0 += RG) take_row(*reinterpret_cast<const u32x4*>(base + (int64_t)r0 * D));  // the block's last rows
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    if (SUM) red[rg][cv * VEC + e] = acc[e];
    if (MAX) redm[rg][cv * VEC + e] = mx[e];
  }
  __syncthreads();
  if (tid < D) {
    const int d = tid;
    double s = 0.0;
    float m = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      if (SUM) s += red[g][d];
      if (MAX) m = fmaxf(m, redm[g][d]);
    }
    const double mean = s / (double)Bs;
    const double val = MODE == 0 ? mean : MODE == 1 ? (double)m : mean + (double)m;
    a.kbar64[blk * D + d] = val;
    const float m32 = (float)val;
    a.kbar32[blk * D + d] = m32;
    const bf16 hi = to_bf16(m32);
    a.kbar_hi[blk * D + d] = hi;
    a.kbar_lo[blk * D + d] = to_bf16(m32 - (float)hi);
    sq[d] = val * val;
  }
  __syncthreads();
  for (int w = D / 2; w > 0; w >>= 1) {
    if (tid < w) sq[tid] += sq[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    const float nrm = (float)(sqrt(sq[0]) * (1.0 + 1e-6));
    a.norm[blk] = nrm;
  }
  // Every query head that reads this key/value head keeps its own list.
  const int64_t heads = a.kv_heads * a.group;
  for (int g = tid; g < a.group; g += 256) a.count[sa.blk0 * heads + (hk * a.group + g) * sa.nb + j] = 0;
}

template <typename T, int D>
static hipError_t pool_launch_t(const PoolArgs& a, hipStream_t s) {
  KernelTimer t(s, "pool");
  const dim3 grid((unsigned)a.kv_blocks);
  switch (a.pooling) {
    case 0: hipLaunchKernelGGL((pool_kernel<T, D, 4, 0>), grid, dim3(256), 0, s, a); break;
    case 1: hipLaunchKernelGGL((pool_kernel<T, D, 4, 1>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((pool_kernel<T, D, 4, 2>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  if (a.bf16_in)
    return a.head_dim == 128 ? pool_launch_t<bf16, 128>(a, s) : pool_launch_t<bf16, 64>(a, s);
  return a.head_dim == 128 ? pool_launch_t<float, 128>(a, s) : pool_launch_t<float, 64>(a, s);
}

}  // namespace moba
