// Varlen packing of the routed (query, past block) pairs.
//
// After routing, each past block is attended by its own batch of queries,
// the varlen layout the MoBA pages describe for handing the chosen blocks to
// the attention kernel without concatenating them into one long sequence
// («MoBA 复现代码跑不通…» §3.3; the hncyxsy.com MOBA article §3).
//
//  pack_scan    — one workgroup: exclusive scans of the per-block query
//                 counts (list offsets) and of ceil(count / tile_m) (gather
//                 tile starts) over all heads and blocks.
//  pack_scatter — one thread per query: places each of its kept past blocks
//                 into that block's list at offset + rank, where rank came
//                 from the gate's atomic count. Entries are
//                 row*(k_eff-1)+slot, row being the query's global row.
//                 The same launch writes the tile map: one thread per gather
//                 workgroup, its tile, block and list range (see tile_map).
#include "common.h"
#include "launch.h"

namespace moba {

__global__ __launch_bounds__(1024) void pack_scan_kernel(const int32_t* __restrict__ count, int64_t n,
                                                         int tile_m, int32_t* __restrict__ offset,
                                                         int32_t* __restrict__ tile_start) {
  __shared__ int64_t sc[1024];
  __shared__ int64_t st[1024];
  const int tid = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = min<int64_t>(n, tid * per), hi = min<int64_t>(n, lo + per);
  int64_t c_sum = 0, t_sum = 0;
  for (int64_t i = lo; i < hi; ++i) {
    const int32_t c = count[i];
    c_sum += c;
    t_sum += (c + tile_m - 1) / tile_m;
  }
  sc[tid] = c_sum;
  st[tid] = t_sum;
  __syncthreads();
  // Inclusive Hillis-Steele scan over the 1024 per-thread totals.
  for (int w = 1; w < 1024; w <<= 1) {
    const int64_t a = tid >= w ? sc[tid - w] : 0;
    const int64_t b = tid >= w ? st[tid - w] : 0;
    __syncthreads();
    sc[tid] += a;
    st[tid] += b;
    __syncthreads();
  }
  int64_t c_run = tid ? sc[tid - 1] : 0, t_run = tid ? st[tid - 1] : 0;
  for (int64_t i = lo; i < hi; ++i) {
    offset[i] = (int32_t)c_run;
    tile_start[i] = (int32_t)t_run;
    const int32_t c = count[i];
    c_run += c;
    t_run += (c + tile_m - 1) / tile_m;
  }
  if (tid == 1023) {
    offset[n] = (int32_t)sc[1023];
    tile_start[n] = (int32_t)st[1023];
  }
}

// Gather workgroup w's tile and that tile's block, list range and sequence,
// so the gather kernel starts with one load. Tiles are dealt to workgroups
// so that each of the 8 XCDs (workgroups go round robin over them) gets one
// contiguous range of tiles, which keeps a block's K/V in one L2:
// tile L = (w % 8) * chunk + w / 8.
__device__ void tile_map(const PackArgs& a, int64_t w) {
  const int64_t nblk = a.q_blocks;
  const int64_t total = a.tile_start[nblk];
  const int64_t chunk = (total + 7) / 8;
  const int64_t li = w / 8, L = (w % 8) * chunk + li;
  int32_t* out = a.tile_map + 4 * w;
  if (li >= chunk || L >= total) {
    out[0] = -1;
    out[1] = out[2] = out[3] = 0;
    return;
  }
  int64_t lo = 0, hi = nblk;  // the last block with tile_start <= L
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (a.tile_start[mid] <= L) lo = mid;
    else hi = mid;
  }
  const int32_t e0 = a.offset[lo] + (int32_t)(L - a.tile_start[lo]) * a.tile_m;
  const int32_t e1 = min(a.offset[lo + 1], e0 + a.tile_m);
  out[0] = (int32_t)lo;
  out[1] = e0;
  out[2] = e1;
  out[3] = (int32_t)seq_find(a.sq, kSeqBlk, a.heads, lo, a.block_size);
}

// One thread per query row (global: sequence, head, token): each kept past
// block's list gets the entry row * (k_eff - 1) + slot at offset + rank.
__global__ __launch_bounds__(256) void pack_scatter_kernel(PackArgs a) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q < a.grid) tile_map(a, q);
  if (q >= a.rows) return;
  const int64_t si = seq_find(a.sq, kSeqTok, a.heads, q, a.block_size);
  const SeqAt sa = seq_at(a.sq, si, a.block_size);
  const int64_t r = q - a.heads * sa.tok0;
  const int64_t h = r / sa.len, t = r % sa.len;
  const int c = (int)(t / a.block_size);
  const int slots = a.k_eff - 1;
  const int32_t* row = a.block_idx + q * a.top_k;
  const int32_t* rk = a.rank + q * slots;
  const int64_t blk0 = sa.blk0 * a.heads + h * sa.nb;  // this head's first block
  const int cap = past_cap(c, sa.nb, a.causal, a.k_eff);
  int s = 0;
  for (int i = 0; i < a.top_k && s < cap; ++i) {
    const int j = row[i];
    if (j < 0) break;
    if (!routed_past_block(j, c, sa.nb, a.causal)) continue;
    a.qlist[a.offset[blk0 + j] + rk[s]] = (int32_t)(q * slots + s);
    ++s;
  }
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  const int64_t n = a.q_blocks;
  {
    KernelTimer t(s, "pack_scan");
    hipLaunchKernelGGL(pack_scan_kernel, dim3(1), dim3(1024), 0, s, a.count, n, a.tile_m, a.offset,
                       a.tile_start);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nt = a.rows > a.grid ? a.rows : a.grid;  // threads: query rows and tile-map entries
  {
    KernelTimer t(s, "pack_scatter");
    hipLaunchKernelGGL(pack_scatter_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moba
