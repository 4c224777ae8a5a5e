// Block mean-pooling of K (the gate's block summary).
//
// The gate of MoBA scores each block by the inner product of the query with
// the mean of the block's keys along the sequence («月之暗面 MoBA 论文解读»
// §3.1, gating.score_fn = mean_pool; the hncyxsy.com MOBA article §3).
//
// Two passes, both bound by HBM bandwidth:
//  pool_partial  — one workgroup per (head, run of R rows); 16-byte loads,
//                  fp64 accumulation per thread, a fixed-order LDS reduction
//                  across row groups; writes a fp64 partial sum per run.
//  pool_finalize — one workgroup per (head, block): sums the block's runs in
//                  order, divides by block_size, and writes the pooled key in
//                  fp64 (exact re-scoring), fp32, and as a bf16 hi/lo pair
//                  (hi = bf16(x), lo = bf16(x - hi)) for the MFMA gate, plus
//                  the block's L2 norm (rounded up) and the head's largest
//                  block norm, for the gate's rounding bound.
// K is read exactly once; fixed reduction orders keep results bit-stable.
#include "common.h"
#include "launch.h"

namespace moba {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_partial_kernel(const T* __restrict__ k,
                                                           double* __restrict__ psum,
                                                           int64_t seq_len, int rows_per_run) {
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int TPR = D / VEC;         // threads per row
  constexpr int RG = 256 / TPR;        // rows per pass
  __shared__ double red[RG][D];
  const int tid = threadIdx.x;
  const int rg = tid / TPR, cv = tid % TPR;
  const int64_t runs_per_head = seq_len / rows_per_run;
  const int64_t bh = blockIdx.x / runs_per_head;
  const int64_t run = blockIdx.x % runs_per_head;
  const T* base = k + (bh * seq_len + run * rows_per_run) * D + cv * VEC;
  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  for (int r = rg; r < rows_per_run; r += RG) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(base + (int64_t)r * D);
    if constexpr (sizeof(T) == 2) {
      const unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)__uint_as_float(w[e] << 16);
        acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
      acc[0] += (double)__uint_as_float(raw.x);
      acc[1] += (double)__uint_as_float(raw.y);
      acc[2] += (double)__uint_as_float(raw.z);
      acc[3] += (double)__uint_as_float(raw.w);
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[rg][cv * VEC + e] = acc[e];
  __syncthreads();
  for (int d = tid; d < D; d += 256) {
    double s = 0.0;
#pragma unroll
    for (int g = 0; g < RG; ++g) s += red[g][d];
    psum[blockIdx.x * (int64_t)D + d] = s;
  }
}

template <int D>
__global__ __launch_bounds__(D) void pool_finalize_kernel(const double* __restrict__ psum,
                                                          int runs_per_block, int64_t block_size,
                                                          double* __restrict__ kbar64,
                                                          float* __restrict__ kbar32,
                                                          bf16* __restrict__ kbar_hi,
                                                          bf16* __restrict__ kbar_lo,
                                                          float* __restrict__ norm,
                                                          unsigned* __restrict__ normmax,
                                                          int64_t n_blocks) {
  __shared__ double red[D];
  const int d = threadIdx.x;
  const int64_t blk = blockIdx.x;  // (bh * n_blocks + j)
  const double* src = psum + blk * runs_per_block * D + d;
  double s = 0.0;
  for (int r = 0; r < runs_per_block; ++r) s += src[(int64_t)r * D];
  const double mean = s / (double)block_size;
  kbar64[blk * D + d] = mean;
  const float m32 = (float)mean;
  kbar32[blk * D + d] = m32;
  const bf16 hi = to_bf16(m32);
  kbar_hi[blk * D + d] = hi;
  kbar_lo[blk * D + d] = to_bf16(m32 - (float)hi);
  red[d] = mean * mean;
  __syncthreads();
  for (int w = D / 2; w > 0; w >>= 1) {
    if (d < w) red[d] += red[d + w];
    __syncthreads();
  }
  if (d == 0) {
    const float nrm = (float)(sqrt(red[0]) * (1.0 + 1e-6));
    norm[blk] = nrm;
    // Non-negative floats order like their bit patterns: an integer max is
    // the float max, independent of the order the blocks finish in.
    atomicMax(normmax + blk / n_blocks, __float_as_uint(nrm));
  }
}

template <typename T, int D>
static hipError_t pool_launch_t(const PoolArgs& a, hipStream_t s) {
  const int64_t runs = a.bh * (a.seq_len / a.rows_per_run);
  {
    KernelTimer t(s, "pool_partial");
    hipLaunchKernelGGL((pool_partial_kernel<T, D>), dim3((unsigned)runs), dim3(256), 0, s,
                       (const T*)a.k, a.psum, a.seq_len, a.rows_per_run);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nblk = a.bh * (a.seq_len / a.block_size);
  {
    KernelTimer t(s, "pool_finalize");
    hipLaunchKernelGGL((pool_finalize_kernel<D>), dim3((unsigned)nblk), dim3(D), 0, s, a.psum,
                       (int)(a.block_size / a.rows_per_run), a.block_size, a.kbar64, a.kbar32,
                       a.kbar_hi, a.kbar_lo, a.norm, a.normmax, a.seq_len / a.block_size);
  }
  return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  if (a.bf16_in)
    return a.head_dim == 128 ? pool_launch_t<bf16, 128>(a, s) : pool_launch_t<bf16, 64>(a, s);
  return a.head_dim == 128 ? pool_launch_t<float, 128>(a, s) : pool_launch_t<float, 64>(a, s);
}

}  // namespace moba
