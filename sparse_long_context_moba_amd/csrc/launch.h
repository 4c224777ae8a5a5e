// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moba {

typedef __bf16 bf16;

// The sequences one launch covers: a batch of equal-length sequences
// (tab == nullptr: every sequence has `len` tokens) or a varlen batch whose
// per-sequence prefix sums sit in a small device table. Tensors hold the
// sequences back to back, sequence i as [heads, len_i, ...] from token
// offset tok0_i, so a query head's row of token t is tok0_i * heads +
// h * len_i + t, and per-block arrays number the blocks of sequence i from
// blk0_i * heads + h * nb_i (nb_i = ceil(len_i / block_size)).
// Table row i (0 <= i <= n) holds the sums over the sequences before i;
// row n holds the totals.
enum SeqCol { kSeqTok = 0, kSeqBlk = 1, kSeqW128 = 2, kSeqW1024 = 3, kSeqW256 = 4 };
constexpr int kSeqCols = 8;
struct Seqs {
  const int64_t* tab;  // [(n + 1) * kSeqCols] or nullptr (uniform)
  int64_t n;           // sequences
  int64_t len;         // tokens per sequence when uniform
};

// Units of column col for one sequence of len tokens.
__host__ __device__ __forceinline__ int64_t seq_units(int col, int64_t len, int64_t block_size) {
  switch (col) {
    case kSeqTok: return len;
    case kSeqBlk: return (len + block_size - 1) / block_size;
    case kSeqW128: return (len + 127) / 128;
    case kSeqW256: return (len + 255) / 256;
    default: return (len + 1023) / 1024;
  }
}
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
  Seqs sq;           // the sequences (k is [tokens of sequence i][kv_heads] head-major per sequence)
  int64_t kv_heads, block_size;
  int64_t kv_blocks;  // kv_heads * total blocks: the launch's work items
  int head_dim;
  bool bf16_in;
  int pooling;       // moba_pooling_t: mean, max, or mean + max per coordinate
  double* kbar64;    // [kv blocks, D]
  float* kbar32;     // [kv blocks, D]
  bf16* kbar_hi;     // [kv blocks, D]
  bf16* kbar_lo;     // [kv blocks, D]
  float* norm;       // [kv blocks] L2 norm of each pooled key, rounded up
  int32_t* count;    // [query-head blocks] the gate's per-block query counts: the pool zeroes them
  int group;         // query heads per key/value head
};
hipError_t launch_pool(const PoolArgs& a, hipStream_t s);

struct GateArgs {
  const void* q;
  const double* kbar64;
  const float* kbar32;
  const bf16* kbar_hi;
  const bf16* kbar_lo;
  const float* norm;   // [kv blocks] L2 norm of each pooled key, rounded up
  Seqs sq;             // the sequences
  int64_t heads, kv_heads, block_size;
  int64_t max_nb;      // most blocks of any sequence (LDS bins of the rank kernel)
  int64_t gate_wgs;    // workgroups of the gate: (kv_heads if shared else heads) * sum ceil(len / 128)
  int64_t gate_wgs256; // the same for 256-query workgroups: heads * sum ceil(len / 256)
  int64_t rank_wgs;    // workgroups of the rank kernel: heads * sum ceil(len / 1024)
  int head_dim;
  bool bf16_in;
  bool causal;
  int top_k;        // columns of block_idx
  int k_eff;        // min(top_k, n_blocks of the longest sequence) (see api.cpp)
  int32_t* block_idx;  // [query rows, top_k]
  int32_t* count;      // [query-head blocks], zeroed before the launch
  int32_t* rank;       // [query rows, k_eff - 1]: position of (row, slot) in its block's list
  int group;           // query heads per key/value head
  bool shared;         // the group routes once, on the sum of its heads' scores
  // Uniform batch fields, read only by the backward's ordered ranks:
  int64_t bh, seq_len, n_blocks;
};
hipError_t launch_gate(const GateArgs& a, hipStream_t s);

struct PackArgs {
  Seqs sq;                    // the sequences
  int64_t heads, block_size;
  int64_t rows;               // query rows: heads * total tokens
  int64_t q_blocks;           // query-head blocks: heads * total blocks
  bool causal;
  int top_k, k_eff;
  int tile_m;                 // queries per gather tile
  const int32_t* block_idx;   // [rows, top_k]
  const int32_t* count;       // [q_blocks]
  const int32_t* rank;        // [rows, k_eff - 1]
  int32_t* offset;            // [q_blocks + 1] exclusive scan of count
  int32_t* tile_start;        // [q_blocks + 1] exclusive scan of ceil(count / tile_m)
  int32_t* qlist;             // [pairs]: row * (k_eff - 1) + slot (row: global query row)
  int64_t grid;               // gather workgroups (a multiple of 8)
  int32_t* tile_map;          // [grid][4]: per gather workgroup {block, e0, e1, sequence}, block -1 if idle
};
hipError_t launch_pack(const PackArgs& a, hipStream_t s);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  Seqs sq;                    // the sequences
  int64_t heads, block_size;
  int64_t diag_wgs;           // own-block (or dense) workgroups: heads * sum ceil(len / 128)
  int head_dim;
  bool bf16_in;
  bool causal;
  int k_eff;
  // gather (past blocks)
  const int32_t* qlist;
  const int32_t* tile_map;    // see PackArgs
  int64_t gather_grid;        // gather workgroups
  void* part_o;               // [query rows, k_eff - 1, D] in the input dtype, lane-native order
  float* part_lse;            // [query rows, k_eff - 1], log2 domain
  int group;                  // query heads per key/value head
  float* lse_out;             // optional [query rows]: natural-log log-sum-exp per query (own-block kernel)
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
  bf16* dq_part;               // [bh, S, k_eff - 1, D] past-block dq partials (bf16, as the forward's)
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
