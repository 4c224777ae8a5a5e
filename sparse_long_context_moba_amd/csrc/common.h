// Shared device types and helpers for the gfx950 MoBA kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moba {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
// Native vector types for raw 16/8-byte moves (HIP's uint4 is a struct
// whose copies can defeat register promotion).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxSlots = 16;  // max past blocks per query outside "keep all" mode

// ----------------------------------------------------------------- MFMA
// Lane layouts (checked on gfx950 with integer-valued operands):
//  32x32x16 bf16: A[i = l%32][k = 8*(l/32) + e], B[k = 8*(l/32) + e][j = l%32],
//                 C[i = 8*(r/4) + 4*(l/32) + r%4][j = l%32], e < 8, r < 16.
//  32x32x2 f32:   A[i = l%32][k = l/32], B[k = l/32][j = l%32], C as above.
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row index inside a 32x32 C tile held in accumulator element r of lane half h.
__device__ __forceinline__ constexpr int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float shfl_xor32(float x) { return __shfl_xor(x, 32); }
__device__ __forceinline__ int shfl_xor32(int x) { return __shfl_xor(x, 32); }
__device__ __forceinline__ double shfl_xor32(double x) { return __shfl_xor(x, 32); }

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_base + 16*l, lds_base being wave-uniform.
// Issued from inline assembly so that the compiler does not make unrelated
// LDS reads wait for it (the builtin form is followed by a full vmcnt wait
// wherever an LDS read of the same array comes later, which would serialise
// the K-ahead stream); the caller waits explicitly (lds_dma_wait) before
// the barrier that publishes the data. The instruction takes its LDS
// address from M0: it is passed as an input operand bound to M0, so the
// compiler itself writes M0 before the instruction and knows its value.
// The instruction has no register outputs (the data goes to LDS), so no
// output register can be reused while the load is in flight.
__device__ __forceinline__ void lds_dma16(const void* src, unsigned lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_base) : "memory");
}
// The same with a wave-uniform base address (SGPR pair) and a 32-bit
// per-lane byte offset, so no per-load 64-bit address arithmetic.
__device__ __forceinline__ void lds_dma16_s(const void* base, unsigned off, unsigned lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void lds_dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Waits until at most N vector memory operations of this wave are in
// flight (they complete in issue order), leaving the newest N running.
template <int N>
__device__ __forceinline__ void lds_dma_wait_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ unsigned lds_addr(const char* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ float bf16_to_f32(unsigned short u) {
  return __uint_as_float(((unsigned)u) << 16);
}

// Round to nearest even fp32 -> bf16 (inputs here are finite).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

// Whether entry j of a block_idx row of a query in block c names a past
// block that query attends: a valid index other than its own block, and
// not a later block under causal routing. Every kernel that turns a
// block_idx row into list entries (ranks, counts, scatter, the backward's
// partial count) skips entries failing this test in the same way and takes
// at most past_cap of them (the first ones; a -1 ends the row), so no row,
// even one edited by a caller, yields more list entries than the exact
// pair count the workspace is sized for.
__device__ __forceinline__ bool routed_past_block(int j, int c, int64_t n_blocks, bool causal) {
  return j >= 0 && j < n_blocks && j != c && (!causal || j < c);
}
// Past blocks a query in block c keeps: min(k_eff - 1, eligible blocks).
__device__ __forceinline__ int past_cap(int c, int64_t n_blocks, bool causal, int k_eff) {
  return min(k_eff - 1, causal ? c : (int)n_blocks - 1);
}

// ------------------------------------------------------------ sequences
// (Seqs and its columns are declared in launch.h.)
// Column col of table row i (the sum over sequences before i).
__device__ __forceinline__ int64_t seq_prefix(const Seqs& s, int64_t i, int col, int64_t block_size) {
  return s.tab ? s.tab[i * kSeqCols + col] : i * seq_units(col, s.len, block_size);
}
// The sequence owning work item `item` when sequence i owns items
// [per * P_i, per * P_{i+1}) of column col (per = heads, for one item per
// head and unit). Uniform: a division; varlen: a binary search.
__device__ __forceinline__ int64_t seq_find(const Seqs& s, int col, int64_t per, int64_t item, int64_t block_size) {
  if (!s.tab) return item / (per * seq_units(col, s.len, block_size));
  int64_t lo = 0, hi = s.n;  // invariant: per * P_lo <= item < per * P_hi
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (per * s.tab[mid * kSeqCols + col] <= item) lo = mid;
    else hi = mid;
  }
  return lo;
}
struct SeqAt {
  int64_t tok0, len, blk0, nb;
};
__device__ __forceinline__ SeqAt seq_at(const Seqs& s, int64_t i, int64_t block_size) {
  SeqAt r;
  r.tok0 = seq_prefix(s, i, kSeqTok, block_size);
  r.len = s.tab ? s.tab[(i + 1) * kSeqCols + kSeqTok] - r.tok0 : s.len;
  r.blk0 = seq_prefix(s, i, kSeqBlk, block_size);
  r.nb = (r.len + block_size - 1) / block_size;
  return r;
}

// A value the whole wave holds alike, marked so for the compiler (a value
// loaded from the sequence table is otherwise taken as per-lane, which
// turns the branches that depend on it into masked ones and defeats the
// instruction scheduling of the loops behind them).
__device__ __forceinline__ int64_t wave_uniform(int64_t x) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const int hi = __builtin_amdgcn_readfirstlane((int)(x >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
// seq_find and seq_at for a work item the whole workgroup shares.
__device__ __forceinline__ int64_t seq_find_u(const Seqs& s, int col, int64_t per, int64_t item, int64_t block_size) {
  return wave_uniform(seq_find(s, col, per, wave_uniform(item), block_size));
}
__device__ __forceinline__ SeqAt seq_at_u(const Seqs& s, int64_t i, int64_t block_size) {
  const SeqAt r = seq_at(s, wave_uniform(i), block_size);
  return SeqAt{wave_uniform(r.tok0), wave_uniform(r.len), wave_uniform(r.blk0), wave_uniform(r.nb)};
}
__device__ __forceinline__ int64_t seq_prefix_u(const Seqs& s, int64_t i, int col, int64_t block_size) {
  return wave_uniform(seq_prefix(s, wave_uniform(i), col, block_size));
}

template <typename T>
struct io;
template <>
struct io<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f(float x) { return x; }
};

}  // namespace moba
