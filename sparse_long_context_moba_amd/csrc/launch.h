// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moba {

typedef __bf16 bf16;

// Past blocks one query may keep when top_k < n_blocks (register top-k limit).
constexpr int kMaxSlotsHost = 16;

// Optional per-kernel event timing (enabled through moba_timing_enable).
// Records a begin event at construction and an end event at destruction on
// the launching stream; does nothing while timing is off.
struct KernelTimer {
  KernelTimer(hipStream_t s, const char* name);
  ~KernelTimer();
  hipStream_t stream;
  int slot;
};

struct PoolArgs {
  const void* k;
  int64_t bh, seq_len, block_size;
  int head_dim;
  bool bf16_in;
  int pooling;       // moba_pooling_t: mean, max, or mean + max per coordinate
  double* kbar64;    // [bh * nb, D]
  float* kbar32;     // [bh * nb, D]
  bf16* kbar_hi;     // [bh * nb, D]
  bf16* kbar_lo;     // [bh * nb, D]
  float* norm;       // [bh * nb] L2 norm of each pooled key, rounded up
  int32_t* count;    // [bh * group * nb] the gate's per-block query counts: the pool zeroes them
  int group;         // query heads per key/value head (bh counts key/value heads here)
};
hipError_t launch_pool(const PoolArgs& a, hipStream_t s);

struct GateArgs {
  const void* q;
  const double* kbar64;
  const float* kbar32;
  const bf16* kbar_hi;
  const bf16* kbar_lo;
  const float* norm;  // [bh * nb] L2 norm of each pooled key, rounded up
  int64_t bh, seq_len, block_size, n_blocks;
  int head_dim;
  bool bf16_in;
  bool causal;
  int top_k;        // columns of block_idx
  int k_eff;        // min(top_k, n_blocks)
  int32_t* block_idx;  // [bh, S, top_k]
  int32_t* count;      // [bh * nb], zeroed before the launch
  int32_t* rank;       // [bh, S, k_eff - 1]: position of (t, slot) in its block's list
  int group;           // query heads per key/value head: query head bh pools key head bh / group
  bool shared;         // the group routes once, on the sum of its heads' scores
};
hipError_t launch_gate(const GateArgs& a, hipStream_t s);

struct PackArgs {
  int64_t bh, seq_len, block_size, n_blocks;
  bool causal;
  int top_k, k_eff;
  int tile_m;                 // queries per gather tile
  const int32_t* block_idx;   // [bh, S, top_k]
  const int32_t* count;       // [bh * nb]
  const int32_t* rank;        // [bh, S, k_eff - 1]
  int32_t* offset;            // [bh * nb + 1] exclusive scan of count
  int32_t* tile_start;        // [bh * nb + 1] exclusive scan of ceil(count / tile_m)
  int32_t* qlist;             // [pairs]: t * (k_eff - 1) + slot
  int64_t grid;               // gather workgroups (a multiple of 8)
  int32_t* tile_map;          // [grid][4]: per gather workgroup {block, e0, e1, 0}, block -1 if idle
};
hipError_t launch_pack(const PackArgs& a, hipStream_t s);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t bh, seq_len, block_size, n_blocks;
  int head_dim;
  bool bf16_in;
  bool causal;
  int k_eff;
  // gather (past blocks)
  const int32_t* qlist;
  const int32_t* tile_map;    // see PackArgs
  int64_t gather_grid;        // gather workgroups
  void* part_o;               // [bh, S, k_eff - 1, D] in the input dtype, lane-native order
  float* part_lse;            // [bh, S, k_eff - 1], log2 domain
  int group;                  // query heads per key/value head: k, v of query head bh are head bh / group
  float* lse_out;             // optional [bh, S]: natural-log log-sum-exp per query (own-block kernel)
};
constexpr int kGatherTileM = 128;
// Gather workgroups for a bound on the number of tiles (a multiple of the
// 8 XCDs, see tile_map_kernel).
constexpr int64_t gather_grid_for(int64_t max_tiles) { return (max_tiles + 7) / 8 * 8; }
hipError_t launch_gather(const AttnArgs& a, hipStream_t s);
hipError_t launch_diag_merge(const AttnArgs& a, hipStream_t s);
hipError_t launch_dense(const AttnArgs& a, hipStream_t s);

// Backward (bf16 inputs): gradients with the forward's block choice fixed.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;            // [bh, S] natural-log log-sum-exp from the forward
  void* dq;                    // [bh, S, D]
  void* dk;                    // [bh / group, S, D]
  void* dv;                    // [bh / group, S, D]
  int64_t bh, seq_len, block_size, n_blocks;
  int head_dim;
  bool causal;
  int k_eff;
  int group;                   // query heads per key/value head
  const int32_t* block_idx;    // [bh, S, top_k] the forward's block choice
  int top_k;                   // columns of block_idx
  const int32_t* qlist;        // per-block query lists (as for the forward's gather)
  const int32_t* offset;       // [bh * nb + 1] list offsets
  const int32_t* tile_map;     // gather tiles
  int64_t gather_grid;
  float* delta;                // [bh, S] do . o
  float* lse2;                 // [bh, S] log-sum-exp in the log2 domain
  float* dq_part;              // [bh, S, k_eff - 1, D] past-block dq partials
  int32_t* lt;                 // [pairs] per list position: the query row
  float* ll;                   // [pairs] its log-sum-exp (log2 domain)
  float* ld;                   // [pairs] its delta
};
hipError_t launch_backward(const BwdArgs& a, hipStream_t s);
// Ranks of a given block_idx in a fixed order, and the per-block counts
// (a.count), for the backward; chunk_counts: [bh, ceil(S / rank_chunk(S)),
// nb] int32 scratch. Needs n_blocks <= 16384. Queries per chunk: 256 while
// a sequence has at most 128 chunks (more waves for short sequences), else
// 1024 (bounded scratch and scan length for long ones); a multiple of 64, so
// the rank order, by 64-query group, does not depend on it.
inline int64_t rank_chunk(int64_t seq_len) { return seq_len <= 128 * 256 ? 256 : 1024; }
hipError_t launch_rank(const GateArgs& a, hipStream_t s, int32_t* chunk_counts);

}  // namespace moba
