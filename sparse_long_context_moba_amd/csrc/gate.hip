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
// a wave 32 of them; for long sequences 256 and 64, two 32-query groups per
// wave (a wave's queries share c because block_size is a multiple of 64).
// Tiles of 32 pooled keys are staged in LDS once per workgroup (two or
// three buffers), one barrier per tile. Scores come from bf16 MFMA 32x32x16 with
// the pooled keys as the A operand (rows = blocks) and the queries as the
// B operand (columns = queries), so lane l holds 16 block scores of query
// l%32. The pooled keys enter as a bf16 hi/lo pair (two MFMA passes, fp32
// accumulate); fp32 inputs use fp32 MFMA on the fp32 means. A gate shared
// by a group of query heads scores the group's summed query (fp32, split
// into a bf16 hi/lo pair: three MFMA passes). The MFMAs of
// tile i+1 are interleaved in the instruction stream with the selection
// work of tile i (waves issue in order).
//
// Selection: each lane keeps the top-TT of its own scores as sortable keys:
// within a segment of 8 tiles as fp32 keys carrying their position in the
// low mantissa bits (insertion = one max and TT-1 med3, independent of each
// other), merged at the segment end into fp64 keys carrying the block index
// (exact, see score_key). The two lane halves merge their lists at the end.
//
// Exactness: every fast score carries a rounding bound
//   eps = gamma * ||q_t||_2 * max_j ||kbar_j||_2   (Cauchy-Schwarz),
// gamma covering the hi/lo residual, the fp32 accumulation and the segment
// key truncation. If the gap
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
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moba {

namespace {

constexpr int kNoBlock = 0x7fffffff;
constexpr int kTileB = 32;          // pooled keys per LDS tile
constexpr int kLdsBinsMax = 8192;   // per-workgroup histogram bins kept in LDS
constexpr int kRankQ = 1024;        // queries per rank workgroup

// Strict order: higher score first, then lower block index.
__device__ __forceinline__ bool better64(double s1, int j1, double s2, int j2) {
  return s1 > s2 || (s1 == s2 && j1 < j2);
}

// Insert (s, j) into a list sorted by `better64`, keeping its length.
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

// Sortable keys for the fast top-k. A fast score s (fp32) converts exactly
// to fp64, which leaves the low 29 mantissa bits zero; the block index goes
// there. Keys of distinct scores keep the scores' order (the index is below
// one fp32 ulp), keys of equal scores differ, and both parts come back
// exactly, so a descending list of keys is kept with fp64 max/min alone:
// inserting key x walks the list with L[i], x = max(L[i], x), min(L[i], x).
// (s = +-0 gives subnormal keys, which fp64 compares keep.) Equal fast
// scores are ordered by index here in either direction; a tie in the fast
// scores is always inside the rounding band, so it is settled by the fp64
// re-scoring below, with the lower index first.
constexpr unsigned kKeyIdxMask = 0x1fffffffu;
// Below every score key (about -2^1023; its index part marks "no block").
constexpr double kKeyNone = __builtin_bit_cast(double, 0xffe000001fffffffull);

__device__ __forceinline__ double score_key(float s, int j) {
  u32x2 b = __builtin_bit_cast(u32x2, (double)s);
  b.x += (unsigned)j;
  return __builtin_bit_cast(double, b);
}
__device__ __forceinline__ float key_score(double k) {
  u32x2 b = __builtin_bit_cast(u32x2, k);
  b.x &= ~kKeyIdxMask;
  return (float)__builtin_bit_cast(double, b);
}
__device__ __forceinline__ int key_block(double k) {
  const unsigned j = __builtin_bit_cast(u32x2, k).x & kKeyIdxMask;
  return j == kKeyIdxMask ? kNoBlock : (int)j;
}
template <int N>
__device__ __forceinline__ void insert_key(double (&L)[N], double x) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const double hi = __builtin_fmax(L[i], x);
    x = __builtin_fmin(L[i], x);
    L[i] = hi;
  }
}

// Segment keys. The scan runs in segments of kSegTiles tiles; within one, a
// lane's scores become fp32 keys whose low kSegBits mantissa bits hold the
// score's position in the segment (tile in segment, accumulator element r;
// the lane half is implicit). Positions are distinct, so keys are distinct
// and order like the truncated scores (truncation moves a score by less
// than 2^-16 of itself, which the rounding bound covers). Inserting x into
// a descending list S is then S'[0] = max(S[0], x), S'[i] = med3(S[i-1],
// S[i], x): one independent operation per slot. At the end of a segment the
// lane's surviving keys are decoded and merged into its fp64 key list.
constexpr int kSegTiles = 8;
constexpr int kSegBits = 7;  // 3 bits of tile, 4 of accumulator element
constexpr unsigned kSegMask = (1u << kSegBits) - 1;
static_assert((kSegTiles << 4) == (1 << kSegBits), "segment position bits");

template <int QG, int TT, bool MASK>
__device__ __forceinline__ void absorb(float (&S)[QG][TT], const f32x16 (&acc)[QG], int tis, int jb, int jend,
                                       int c) {
  const unsigned pos0 = (unsigned)tis << 4;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const unsigned pos = pos0 + r;
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      // The element is read as a scalar first: this compiler turns
      // __builtin_bit_cast of a vector element into a cast of element 0.
      const float sv = acc[g][r];
      float x = __uint_as_float((__float_as_uint(sv) & ~kSegMask) | pos);
      if (MASK) {
        const int j = jb + 8 * (r >> 2) + (r & 3);
        x = (j < jend && j != c) ? x : kNegInf;
      }
      float n[TT];
      n[0] = __builtin_fmaxf(S[g][0], x);
#pragma unroll
      for (int i = 1; i < TT; ++i) n[i] = __builtin_amdgcn_fmed3f(S[g][i - 1], S[g][i], x);
#pragma unroll
      for (int i = 0; i < TT; ++i) S[g][i] = n[i];
    }
  }
}

// Moves a segment's keys (segment starting at block seg0) into the fp64 key
// lists and clears the segment lists. h is the lane half.
template <int QG, int TT>
__device__ __forceinline__ void flush_segment(float (&S)[QG][TT], double (&L)[QG][TT], int seg0, int h) {
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const unsigned kb = __builtin_bit_cast(unsigned, S[g][i]);
      const unsigned p = kb & kSegMask, r = p & 15;
      const int j = seg0 + 32 * (int)(p >> 4) + 8 * (int)(r >> 2) + 4 * h + (int)(r & 3);
      const bool empty = S[g][i] == kNegInf;
      // (An empty slot decodes to garbage; it is replaced, not inserted.)
      const float sv = empty ? 0.f : __builtin_bit_cast(float, kb & ~kSegMask);
      const double x = score_key(sv, j);
      insert_key(L[g], empty ? kKeyNone : x);
      S[g][i] = kNegInf;
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
  // Staging of one tile, rows j0 .. j0+31 of hi then lo (rows past the last
  // block repeat it): NLD 16-byte chunks per thread, fetched into registers
  // one tile ahead and stored to LDS after the current tile is scored.
  using Chunk = u32x4;
  static constexpr int CPR = D / 8;             // chunks per row
  static constexpr int CH = kTileB * CPR;       // chunks per tile of hi (or lo)
  static constexpr int NLD = 2 * CH / 256;
  // kvb0: index of the head's first pooled key; nb: the head's blocks.
  static __device__ void fetch(Chunk (&r)[NLD], const GateArgs& a, int64_t kvb0, int nb, int j0, int tid) {
    const int64_t head = kvb0 * D;
    if (j0 + kTileB <= nb) {
      // Whole tile: a uniform base and a fixed per-thread offset.
      const bf16* hi = a.kbar_hi + head + (int64_t)j0 * D;
      const bf16* lo = a.kbar_lo + head + (int64_t)j0 * D;
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int i = tid + 256 * n, id = i % CH;
        r[n] = *reinterpret_cast<const Chunk*>((i < CH ? hi : lo) + (id / CPR) * D + 8 * (id % CPR));
      }
    } else {
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int i = tid + 256 * n, id = i % CH;
        const int j = min(j0 + id / CPR, nb - 1);
        r[n] = *reinterpret_cast<const Chunk*>((i < CH ? a.kbar_hi : a.kbar_lo) + head + (int64_t)j * D + 8 * (id % CPR));
      }
    }
  }
  static __device__ void put(char* lds, const Chunk (&r)[NLD], int tid) {
    bf16* hi = reinterpret_cast<bf16*>(lds);
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int i = tid + 256 * n, which = i / CH, id = i % CH;
      *reinterpret_cast<Chunk*>(hi + which * kTileB * KR + (id / CPR) * KR + 8 * (id % CPR)) = r[n];
    }
  }
  // Direct HBM -> LDS staging instead of fetch/put. A tile is a run of
  // 16-byte slots: rows of RC slots (hi rows, then lo rows), each row's last
  // slot padding, which repeats the row's first chunk. One wave-wide load
  // fills 64 consecutive slots, so the four waves share NDMA_ALL loads; a
  // wave with fewer repeats the last one (same data to the same slots).
  static constexpr bool kDma = true;
  static constexpr int RC = KR / 8;
  static constexpr int SLOTS = 2 * kTileB * RC;
  static constexpr int NDMA_ALL = SLOTS / 64;
  static_assert(SLOTS % 64 == 0 && KR % 8 == 0, "whole wave-wide loads per tile");
  static constexpr int NDMA = (NDMA_ALL + 3) / 4;  // loads per wave per tile
  static __device__ int dma_ins(int w, int n) { return min(w + 4 * n, NDMA_ALL - 1); }
  // Byte offsets of this lane's slots from the tile's first hi row; lo rows
  // lie lo_off bytes further; rows at or past `rows` repeat the last one.
  static __device__ void dma_offsets(unsigned (&off)[NDMA], int w, int lane, unsigned lo_off, int rows) {
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int sl = 64 * dma_ins(w, n) + lane;
      const int row = sl / RC;
      const int ch = sl % RC < D / 8 ? sl % RC : 0;
      const int r = min(row % kTileB, rows - 1);
      off[n] = (row < kTileB ? 0u : lo_off) + (unsigned)r * (D * 2) + 16u * ch;
    }
  }
  static __device__ void dma(const bf16* tile_hi, const unsigned (&off)[NDMA], unsigned lds, int w) {
#pragma unroll
    for (int n = 0; n < NDMA; ++n) lds_dma16_s(tile_hi, off[n], lds + 1024u * dma_ins(w, n));
  }
  // Scores of every group against the tile: each pooled-key fragment is read
  // from LDS once and feeds one MFMA per group (independent chains).
  template <int QG>
  static __device__ void scores(const char* lds, int col, int h, const GateOps (&qf)[QG], f32x16 (&acc)[QG]) {
    const bf16* hi = reinterpret_cast<const bf16*>(lds) + col * KR + 8 * h;
    const bf16* lo = hi + kTileB * KR;
#pragma unroll
    for (int g = 0; g < QG; ++g) acc[g] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(hi + 16 * kk);
#pragma unroll
      for (int g = 0; g < QG; ++g) acc[g] = mfma_bf16(af, qf[g].f[kk], acc[g]);
    }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(lo + 16 * kk);
#pragma unroll
      for (int g = 0; g < QG; ++g) acc[g] = mfma_bf16(af, qf[g].f[kk], acc[g]);
    }
  }
  // The steady state in issue order (waves issue in order, so the MFMA
  // chains only overlap the selection work if the two are interleaved in
  // the instruction stream): scores of the next tile (nxt) from LDS with
  // fragment reads AH ahead, each fragment feeding one MFMA per query
  // group, and between consecutive fragments the fold of 16 / (2 KC) of
  // each group's current scores (cur) into its segment list S. Scheduling
  // fences keep this order.
  template <int QG, int TT>
  static __device__ __forceinline__ void scores_fold(const char* lds, int col, int h, const GateOps (&qf)[QG],
                                                     f32x16 (&nxt)[QG], const f32x16 (&cur)[QG], float (&S)[QG][TT],
                                                     unsigned pos0) {
    const bf16* hi = reinterpret_cast<const bf16*>(lds) + col * KR + 8 * h;
    const bf16* lo = hi + kTileB * KR;
    constexpr int NF = 2 * KC, AH = 4, EPF = 16 / NF;  // fragments, reads ahead, elements folded per fragment
    static_assert(16 % NF == 0, "fold elements split evenly over the fragments");
    auto frag = [&](int c) { return *reinterpret_cast<const bf16x8*>((c < KC ? hi : lo) + 16 * (c % KC)); };
    bf16x8 f[AH];
#pragma unroll
    for (int c = 0; c < AH; ++c) f[c] = frag(c);
#pragma unroll
    for (int g = 0; g < QG; ++g) nxt[g] = f32x16{};
#pragma unroll
    for (int c = 0; c < NF; ++c) {
#pragma unroll
      for (int g = 0; g < QG; ++g) nxt[g] = mfma_bf16(f[c % AH], qf[g].f[c % KC], nxt[g]);
      if (c + AH < NF) f[c % AH] = frag(c + AH);
#pragma unroll
      for (int g = 0; g < QG; ++g)
#pragma unroll
        for (int u = 0; u < EPF; ++u) {
          const int r = EPF * c + u;
          const float sv = cur[g][r];
          const float x = __uint_as_float((__float_as_uint(sv) & ~kSegMask) | (pos0 + r));
          float n[TT];
          n[0] = __builtin_fmaxf(S[g][0], x);
#pragma unroll
          for (int i = 1; i < TT; ++i) n[i] = __builtin_amdgcn_fmed3f(S[g][i - 1], S[g][i], x);
#pragma unroll
          for (int i = 0; i < TT; ++i) S[g][i] = n[i];
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Issue order for the steady state (waves issue in order, so the MFMA
  // chains only overlap the selection work if the two are interleaved in
  // the instruction stream): a few fragment reads ahead, then per fragment
  // its QG MFMAs and an even share of the selection's VALU work.
  template <int QG, int TT>
  static __device__ __forceinline__ void interleave() {
    constexpr int NF = 2 * KC;                     // fragments (hi and lo)
    constexpr int VALU = 16 * QG * (TT + 1) + 16;  // selection work per tile
    constexpr int PER = (VALU + NF - 1) / NF;
    constexpr int AHEAD = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, QG, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
      if (f + AHEAD < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  // Relative rounding bound of a fast score: hi/lo residual (<= 2^-16 of
  // each mean coordinate, taken as 2^-15), 2D+16 fp32 accumulation steps at
  // 2^-22 each (a 4x margin over rounding to nearest) and the segment key
  // truncation (2^-16).
  static __device__ constexpr float gamma() {
    return 3.0517578e-05f + (2 * D + 16) * 2.3841858e-07f + 1.5258789e-05f;
  }
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
  // 8-byte chunks: the padded row stride (D + 2 floats) keeps the column
  // reads conflict-free but leaves odd rows 8-byte aligned.
  using Chunk = u32x2;
  static constexpr int CPR = D / 2;
  static constexpr int CH = kTileB * CPR;
  static constexpr int NLD = CH / 256;
  static __device__ void fetch(Chunk (&r)[NLD], const GateArgs& a, int64_t kvb0, int nb, int j0, int tid) {
    const float* head = a.kbar32 + kvb0 * D;
    if (j0 + kTileB <= nb) {
      const float* base = head + (int64_t)j0 * D;
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int id = tid + 256 * n;
        r[n] = *reinterpret_cast<const Chunk*>(base + (id / CPR) * D + 2 * (id % CPR));
      }
    } else {
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int id = tid + 256 * n;
        const int j = min(j0 + id / CPR, nb - 1);
        r[n] = *reinterpret_cast<const Chunk*>(head + (int64_t)j * D + 2 * (id % CPR));
      }
    }
  }
  // Register staging (8-byte chunks at an odd row stride cannot be
  // loaded straight into LDS 16 bytes at a time).
  static constexpr bool kDma = false;
  static constexpr int NDMA = 1;
  static __device__ void dma_offsets(unsigned (&)[NDMA], int, int, unsigned, int) {}
  static __device__ void dma(const bf16*, const unsigned (&)[NDMA], unsigned, int) {}
  static __device__ void put(char* lds, const Chunk (&r)[NLD], int tid) {
    float* kt = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int id = tid + 256 * n;
      *reinterpret_cast<Chunk*>(kt + (id / CPR) * KR + 2 * (id % CPR)) = r[n];
    }
  }
  static constexpr int QG_MAX = 1;  // the fp32 query fragment alone takes D/2 registers
  template <int QG>
  static __device__ void scores(const char* lds, int col, int h, const GateOps (&qf)[QG], f32x16 (&acc)[QG]) {
    static_assert(QG == 1, "one query group");
    const float* kt = reinterpret_cast<const float*>(lds) + col * KR + h;
    acc[0] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) acc[0] = mfma_f32(kt[2 * kk], qf[0].f[kk], acc[0]);
  }
  template <int QG, int TT>
  static __device__ __forceinline__ void interleave() {
    constexpr int VALU = 16 * QG * (TT + 1) + 16;
    constexpr int PER = (VALU + KC - 1) / KC;
#pragma unroll
    for (int f = 0; f < KC; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, QG, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
    }
  }
  // fp32 products and 2D+16 accumulation steps at 2^-22 each, and the
  // segment key truncation (2^-16).
  static __device__ constexpr float gamma() { return (2 * D + 16) * 2.3841858e-07f + 1.5258789e-05f; }
};

// Shared gate: the group's summed query, taken in fp32 and split into a
// bf16 pair (hi = bf16(x), lo = bf16(x - hi)), against the pooled keys' bf16
// pair: three MFMA products (hi.hi, hi.lo, lo.hi; lo.lo is below 2^-16 of
// the score and left to the rounding bound). The tile staging is the
// per-head bf16 one.
template <int D>
struct GateOpsSplitQ : GateOps<bf16, D> {
  using Base = GateOps<bf16, D>;
  static constexpr int KC = Base::KC, KR = Base::KR;
  bf16x8 f[KC];  // hi
  bf16x8 g[KC];  // lo
  // Sum of the ng query rows (head order) in fp32, split into hi/lo.
  // Returns sum_h ||q_h|| over both lane halves.
  template <typename TQ>
  __device__ float load_sum(const TQ* qrow, int64_t head_stride, int ng, int h) {
    float x[KC][8];
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[kk][e] = 0.f;
    float norms = 0.f;
    for (int gh = 0; gh < ng; ++gh) {
      const TQ* r = qrow + gh * head_stride;
      float ss = 0.f;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = (float)r[16 * kk + 8 * h + e];
          x[kk][e] += y;
          ss = __builtin_fmaf(y, y, ss);
        }
      ss += shfl_xor32(ss);
      norms += __builtin_sqrtf(ss);
    }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16 hi = to_bf16(x[kk][e]);
        f[kk][e] = hi;
        g[kk][e] = to_bf16(x[kk][e] - (float)hi);
      }
    return norms;
  }
  static constexpr int QG_MAX = 1;
  template <int QG>
  static __device__ void scores(const char* lds, int col, int h, const GateOpsSplitQ (&qf)[QG],
                                f32x16 (&acc)[QG]) {
    static_assert(QG == 1, "one query group");
    const bf16* hi = reinterpret_cast<const bf16*>(lds) + col * KR + 8 * h;
    const bf16* lo = hi + kTileB * KR;
    acc[0] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(hi + 16 * kk);
      acc[0] = mfma_bf16(af, qf[0].f[kk], acc[0]);
      acc[0] = mfma_bf16(af, qf[0].g[kk], acc[0]);
    }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(lo + 16 * kk);
      acc[0] = mfma_bf16(af, qf[0].f[kk], acc[0]);
    }
  }
  // Issue order as in the per-head gate: two MFMAs per hi fragment, one per
  // lo fragment, each with an even share of the selection's VALU work.
  template <int QG, int TT>
  static __device__ __forceinline__ void interleave() {
    constexpr int NF = 2 * KC;
    constexpr int VALU = 16 * QG * (TT + 1) + 16;
    constexpr int PER = (VALU + NF - 1) / NF;
    constexpr int AHEAD = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int fr = 0; fr < KC; ++fr) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int fr = KC; fr < NF; ++fr) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
      if (fr + AHEAD < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  // Relative rounding bound: the pooled keys' hi/lo residual, the summed
  // query's hi/lo residual and the omitted lo.lo product (each <= 2^-16,
  // taken as 2^-15), 3D+16 fp32 accumulation steps at 2^-22 each and the
  // segment key truncation (2^-16). The fp32 sum of the heads' queries is
  // added by the caller.
  static __device__ constexpr float gamma() {
    return 3 * 3.0517578e-05f + (3 * D + 16) * 2.3841858e-07f + 1.5258789e-05f;
  }
};

template <bool C, typename A, typename B>
struct pick_type {
  using type = A;
};
template <typename A, typename B>
struct pick_type<false, A, B> {
  using type = B;
};

// Shapes of the per-head bf16 gate with short lists (top_k <= 5), by the
// longest sequence's block count (same-box A/Bs, identical routing):
//  * up to kShortMaxBlocks: one 32-query group per wave, two tile buffers
//    (35 KB of LDS at head_dim 128) and four waves per SIMD, so four
//    workgroups per compute unit; their short scans are bound by load
//    latency (against three buffers at three waves: -9 % at 64 blocks,
//    -13 % at 128, -6 % at 256 and 384; -3 % at 512 against two groups);
//  * above it: two 32-query groups per wave (QG), 256-query workgroups at
//    two waves per SIMD with three buffers and the branch-free stretch.
//    Every pooled-key fragment read from LDS feeds two MFMAs, half the LDS
//    reads per MFMA (-4 % at 2048 blocks against the one-group three-buffer
//    form; the short form is 2 % slower at 1024 blocks and 5 % at 2048).
// The shared gate (two query fragments, hi and lo of the group's summed
// query) takes the short form at three waves per SIMD at every length
// (against three buffers at two waves: -15 % at 64 blocks with top_k 3,
// -11 % with top_k 5, -18 % at 256 blocks, -16 % at 512, -17 % at 1024,
// -19 % at 2048); fp32 gates and longer lists take one group and two waves
// (two buffers for fp32, three else).
template <typename T, int D, int TT, bool SHARED, int QG, int NBUF>
constexpr int gate_waves() {
  return (sizeof(T) == 2 && TT <= 6 && QG == 1 && NBUF == 2) ? (SHARED ? 3 : 4) : 2;
}
constexpr int kShortMaxBlocks = 512;

// Exact top-TT over every eligible block of one query, by the whole wave:
// the query's fp64 vector (D values) is in this wave's LDS slice qs; lane l
// scores blocks l, l + 64, ... as fp64 dot products summed over the
// coordinates in order, and keeps its own top-TT by (score desc, index
// asc). TT rounds of a wave-wide arg-max over the lists' heads (the lane
// holding the winner drops it) then give the overall top-TT in order, the
// same in every lane. One load round trip serves 64 blocks.
template <int D, int TT>
__device__ void rescan_all(const double* kb64, const double* qs, int c, int jend, int lane, int (&top)[TT]) {
  double es[TT];
  int ej[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    es[i] = -__builtin_huge_val();
    ej[i] = kNoBlock;
  }
  for (int j0 = 0; j0 < jend; j0 += 64) {
    const int j = j0 + lane;
    const bool on = j < jend && j != c;
    const double* kr = kb64 + (int64_t)(on ? j : 0) * D;
    double p = 0.0;
#pragma unroll 4
    for (int d = 0; d < D; d += 2) {
      const double2 kv = *reinterpret_cast<const double2*>(kr + d);
      const double2 qv = *reinterpret_cast<const double2*>(qs + d);
      p = __builtin_fma(qv.x, kv.x, p);
      p = __builtin_fma(qv.y, kv.y, p);
    }
    if (on && better64(p, j, es[TT - 1], ej[TT - 1])) insert_full64(es, ej, p, j);
  }
#pragma unroll
  for (int r = 0; r < TT; ++r) {
    double bs = es[0];
    int bj = ej[0];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double os = __shfl_xor(bs, off);
      const int oj = __shfl_xor(bj, off);
      if (better64(os, oj, bs, bj)) {
        bs = os;
        bj = oj;
      }
    }
    top[r] = bj;
    if (bj != kNoBlock && ej[0] == bj) {  // this lane held the winner
#pragma unroll
      for (int i = 0; i + 1 < TT; ++i) {
        es[i] = es[i + 1];
        ej[i] = ej[i + 1];
      }
      es[TT - 1] = -__builtin_huge_val();
      ej[TT - 1] = kNoBlock;
    }
  }
}

// fp64 re-scoring of the wave's ambiguous queries (lanes with `amb` set,
// lane half 0), one query at a time by the whole wave. A query's fp64
// vector is the sum of its rows in nq query heads (one head unless the gate
// is shared): row qrow0 + tg + lane column of the first, the others
// head_stride rows apart; the pooled keys are the key head's, from kvb0.
// The queries share c
// and the eligible set. Candidates are the query's tracked list, or every
// eligible block when its rounding band reaches past the list (`tracked`
// false). For the tracked list, 64 lanes split each candidate's dot product
// into D/8 slices of 8 coordinates and sum the slices in a fixed order
// (deterministic); every eligible block goes through rescan_all, with the
// query in the wave's LDS slice qs (D doubles). The query in lane column L
// gets the exact top-TT in sel.
template <typename TQ, int D, int TT>
__device__ void rescore_ambiguous(const GateArgs& a, int64_t qrow0, int64_t head_stride, int nq, int64_t kvb0,
                                  int64_t tg, int c, int jend, bool amb, bool tracked, const int (&lj)[TT], int (&sel)[TT],
                                  int lane, int col, double* qs) {
  uint64_t pend = __builtin_amdgcn_ballot_w64(amb);
  const double* kb64 = a.kbar64 + kvb0 * (int64_t)D;
  constexpr int SL = D / 8;    // 8-coordinate slices per candidate
  constexpr int G = 64 / SL;   // candidates per pass
  const int gi = lane / SL, sl = lane % SL;
  while (pend) {
    const int ln = __builtin_ctzll(pend);
    pend &= pend - 1;
    const bool trk = __builtin_amdgcn_readlane((int)tracked, ln);
    if (!trk) {
      // The query (summed over its heads in fp64) into the wave's LDS slice,
      // then every eligible block.
      const TQ* qA = reinterpret_cast<const TQ*>(a.q) + (qrow0 + tg + ln) * D;
      for (int d = lane; d < D; d += 64) {
        double x = (double)(float)qA[d];
        for (int g = 1; g < nq; ++g) x += (double)(float)qA[g * head_stride * D + d];
        qs[d] = x;
      }
      int top[TT];
      rescan_all<D, TT>(kb64, qs, c, jend, lane, top);
      if (col == ln) {
#pragma unroll
        for (int i = 0; i < TT; ++i) sel[i] = top[i];
      }
      continue;
    }
    // This lane's slice of the ambiguous query's coordinates, summed over
    // the heads in fp64.
    const TQ* qL = reinterpret_cast<const TQ*>(a.q) + (qrow0 + tg + ln) * D + 8 * sl;
    double qd[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qd[e] = (double)(float)qL[e];
    for (int g = 1; g < nq; ++g) {
      const TQ* qg = qL + g * head_stride * D;
#pragma unroll
      for (int e = 0; e < 8; ++e) qd[e] += (double)(float)qg[e];
    }
    int cj[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) cj[i] = __builtin_amdgcn_readlane(lj[i], ln);
    double es[TT];
    int ej[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      es[i] = -__builtin_huge_val();
      ej[i] = kNoBlock;
    }
    for (int base = 0; base < TT; base += G) {
      const int ci = base + gi;
      int j = kNoBlock;
#pragma unroll
      for (int i = 0; i < TT; ++i)
        if (ci == i) j = cj[i];
      double p = 0.0;
      if (j != kNoBlock) {
        const double* kr = kb64 + (int64_t)j * D + 8 * sl;
#pragma unroll
        for (int e = 0; e < 8; ++e) p = __builtin_fma(qd[e], kr[e], p);
      }
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
    if (col == ln) {
#pragma unroll
      for (int i = 0; i < TT; ++i) sel[i] = ej[i];
    }
  }
}

// Writes one block_idx row: the m kept past blocks and the own block c,
// ascending, padded with -1. Without scoring, either only c (m = 0) or every
// block below jstop (all eligible blocks are kept).
template <int TT>
__device__ void write_row(int32_t* row, const int (&sel)[TT], bool scoring, int m, int c, int jstop, int top_k) {
  int col_out = 0;
  if (!scoring) {
    if (m == 0) {
      row[col_out++] = c;
    } else {
      for (int j = 0; j < jstop; ++j) row[col_out++] = j;
    }
    for (; col_out < top_k; ++col_out) row[col_out] = -1;
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
  bool own_done = false;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    if (i < m) {
      const int j = srt[i];
      if (!own_done && c < j) {
        row[col_out++] = c;
        own_done = true;
      }
      row[col_out++] = j;
    }
  }
  if (!own_done) row[col_out++] = c;
  for (; col_out < top_k; ++col_out) row[col_out] = -1;
}

}  // namespace

// T is the type the scores are computed in (the MFMA path), TQ the stored
// query type. SHARED: one workgroup row of queries per key/value head, the
// scores being those of the group's summed query (bf16 MFMA on its hi/lo
// split, T = bf16).
template <typename T, typename TQ, int D, int TT, bool SHARED, int QG, int NBUF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(gate_waves<T, D, TT, SHARED, QG, NBUF>()))) void
gate_topk_kernel(GateArgs a) {
  using Ops = typename pick_type<SHARED, GateOpsSplitQ<D>, GateOps<T, D>>::type;
  static_assert(!SHARED || sizeof(T) == 2, "a shared gate scores on the bf16 pair");
  static_assert(SHARED || sizeof(T) == sizeof(TQ), "a per-head gate scores in the query's own type");
  static_assert(QG == 1 || (std::is_same<Ops, GateOps<bf16, D>>::value && TT <= 6), "two groups: per-head bf16, short lists");
  constexpr int WQ = 32 * QG;       // queries per wave
  constexpr int WGQ = 4 * WQ;       // queries per workgroup
  constexpr int COL = WGQ == 128 ? kSeqW128 : kSeqW256;
  extern __shared__ __align__(16) char smem[];
  char* tile = smem;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // the wave (uniform)
  static_assert(WGQ == 128 || WGQ == 256, "the sequence table counts gate workgroups of 128 or 256 queries");
  // Work item -> (sequence, routing row, workgroup). Per-head gate: the row
  // is a query head, reading key head row / group. Shared gate: the row is
  // a key/value head and routes its group of query heads.
  const int64_t rows = SHARED ? a.kv_heads : a.heads;
  const int64_t item = blockIdx.x;
  const int64_t si = seq_find_u(a.sq, COL, rows, item, a.block_size);
  const SeqAt sa = seq_at_u(a.sq, si, a.block_size);
  const int64_t wg_per_head = (sa.len + WGQ - 1) / WGQ;
  const int64_t r_item = item - rows * seq_prefix_u(a.sq, si, COL, a.block_size);
  const int64_t grp = r_item / wg_per_head;
  const int64_t kvh = SHARED ? grp : grp / a.group;
  const int64_t qh0 = SHARED ? grp * a.group : grp;
  const int nq = SHARED ? a.group : 1;
  // Within a head, workgroups run latest queries first: they scan the most
  // blocks (causal), so the short ones fill the tail of the launch.
  const int64_t qb = (wg_per_head - 1 - r_item % wg_per_head) * WGQ;
  const int64_t len = sa.len;
  const int64_t qrow0 = sa.tok0 * a.heads + qh0 * len;    // row of token 0 in query head qh0
  const int64_t kvb0 = sa.blk0 * a.kv_heads + kvh * sa.nb;  // the key head's first pooled key
  // The wave's queries t0 .. t0 + WQ - 1 (group g, lane column col: query
  // t0 + 32 g + col) lie in one block, as block_size is a multiple of 64;
  // lanes past the sequence's end (qvalid false) compute on its last query
  // and write nothing.
  const int64_t t0 = qb + WQ * w;
  const bool wave_on = t0 < len;  // workgroup-uniform control flow below
  const int64_t tw = wave_on ? t0 : qb;
  const int NB = (int)sa.nb;
  const int c = (int)(tw / a.block_size);
  const int n_elig = a.causal ? c : NB - 1;
  const int m = min(a.k_eff - 1, n_elig);
  const bool scoring = wave_on && m > 0 && m < n_elig;  // wave-uniform

  // ---- fast scores over the eligible blocks, top-TT per lane half
  Ops qf[QG];
  float qnorm[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    qnorm[g] = 0.f;
    if (scoring) {
      const TQ* qrow = reinterpret_cast<const TQ*>(a.q) + (qrow0 + min<int64_t>(tw + 32 * g + col, len - 1)) * D;
      if constexpr (SHARED) {
        qnorm[g] = qf[g].template load_sum<TQ>(qrow, len * D, nq, h) * 1.0001f;
      } else {
        qf[g].load(qrow, h);
        float qss = qf[g].sumsq();
        qss += shfl_xor32(qss);
        qnorm[g] = __builtin_sqrtf(qss) * 1.0001f;
      }
    }
  }
  const int jend = a.causal ? c : NB;  // this wave's scan bound
  double L[QG][TT];
  float S[QG][TT];
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      L[g][i] = kKeyNone;
      S[g][i] = kNegInf;
    }
  // Scan bound of the whole workgroup (its last valid query has the largest c).
  const int64_t t_last = min<int64_t>(qb + WGQ, len) - 1;
  const int wg_jend = a.causal ? (int)(t_last / a.block_size) : NB;
  // Largest pooled-key norm among the blocks the workgroup scans (each wave
  // scans a prefix of them, so it bounds every wave's norms), for the
  // rounding bound. All threads request their share of the norms at once,
  // 2048 per round trip, next to the first tile's loads; the result is
  // published by the pipeline's first barrier.
  __shared__ float wg_kmax[4];
  __shared__ int wg_full[4];
  {
    const float* nrm = a.norm + kvb0;
    float kpart = 0.f;
    for (int j0 = 0; j0 < wg_jend; j0 += 256 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + 256 * u + tid;
        v[u] = j < wg_jend ? nrm[j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) kpart = fmaxf(kpart, v[u]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) kpart = fmaxf(kpart, __shfl_xor(kpart, off));
    if (lane == 0) {
      wg_kmax[w] = kpart;
      // Leading tiles of this wave's scan that hold no own block and no
      // block past its bound (none if it does not score).
      wg_full[w] = !scoring ? 0 : a.causal ? jend / kTileB : min(jend, c) / kTileB;
    }
  }
  // Tile pipeline. Step i passes a workgroup barrier behind which tile i+1
  // is in LDS, issues the MFMAs of tile i+1 and, while they run, folds the
  // scores of tile i (issued one step earlier) into the key lists. Only the
  // ordering of independent work changes; every tile is scored and folded
  // exactly once.
  //  * bf16 ops load tiles straight into LDS (NBUF buffers, tile t in
  //    buffer t % NBUF): step i waits for its own loads of tile i+1 (with
  //    three buffers issued two steps earlier, leaving tile i+2's in
  //    flight; with two, one step earlier), passes the barrier (all waves'
  //    loads of tile i+1 landed; every wave is done reading tile i, which
  //    its MFMAs read in step i-1) and then loads tile i+NBUF into tile
  //    i's buffer.
  //  * fp32 ops stage through registers (two buffers, tile t in buffer
  //    t & 1): step i stores tile i+1 (fetched one step earlier), passes the
  //    barrier and fetches tile i+2.
  constexpr bool DMA = Ops::kDma;
  static_assert(NBUF == 2 || (DMA && NBUF == 3), "tile buffers: two, or three for direct loads");
  auto buf = [&](int t) { return tile + (t % NBUF) * Ops::TILE_BYTES; };
  const int ntiles = (wg_jend + kTileB - 1) / kTileB;  // workgroup-uniform
  const int my_tiles = scoring ? (jend + kTileB - 1) / kTileB : 0;
  typename Ops::Chunk stg[Ops::NLD];
  unsigned doff[Ops::NDMA];
  const unsigned lo_off = (unsigned)(reinterpret_cast<const char*>(a.kbar_lo) - reinterpret_cast<const char*>(a.kbar_hi));
  auto issue = [&](int t) {  // loads of tile t (bf16 ops)
    const bf16* base = a.kbar_hi + (kvb0 + (int64_t)t * kTileB) * D;
    const int rows = NB - t * kTileB;  // the head's blocks from the tile's first
    if (rows >= kTileB) {
      Ops::dma(base, doff, lds_addr(buf(t)), w);
    } else {
      unsigned po[Ops::NDMA];
      Ops::dma_offsets(po, w, lane, lo_off, rows);
      Ops::dma(base, po, lds_addr(buf(t)), w);
    }
  };
  f32x16 acc_a[QG], acc_b[QG];
  if constexpr (DMA) {
    Ops::dma_offsets(doff, w, lane, lo_off, kTileB);
    for (int t = 0; t < min(ntiles, NBUF); ++t) issue(t);
    if (NBUF == 3 && ntiles >= 3) lds_dma_wait_n<2 * Ops::NDMA>();
    else if (ntiles >= 2) lds_dma_wait_n<Ops::NDMA>();
    else lds_dma_wait();
  } else if (ntiles > 0) {
    Ops::fetch(stg, a, kvb0, NB, 0, tid);
    Ops::put(tile, stg, tid);
  }
  __syncthreads();
  if (!DMA && ntiles > 1) Ops::fetch(stg, a, kvb0, NB, kTileB, tid);
  if (my_tiles > 0) Ops::template scores<QG>(tile, col, h, qf, acc_a);
  auto step = [&](int i, f32x16(&cur)[QG], f32x16(&nxt)[QG]) {
    char* next_buf = buf(i + 1);
    if constexpr (DMA) {
      if (NBUF == 3 && i + 2 < ntiles) lds_dma_wait_n<Ops::NDMA>();
      else lds_dma_wait();
      __syncthreads();
      if (i + NBUF < ntiles) issue(i + NBUF);
    } else {
      if (i + 1 < ntiles) Ops::put(next_buf, stg, tid);
      __syncthreads();
      if (i + 2 < ntiles) Ops::fetch(stg, a, kvb0, NB, (i + 2) * kTileB, tid);
    }
    const bool do_next = i + 1 < my_tiles, do_cur = i < my_tiles;
    const int jt = i * kTileB, tis = i % kSegTiles;
    const int jb = jt + 4 * h;
    const bool full = jt + kTileB <= jend && (a.causal || c < jt || c >= jt + kTileB);
    if (do_cur && do_next && full) {  // the steady state: one basic block
      if constexpr (std::is_same<Ops, GateOps<bf16, D>>::value) {
        // the MFMAs of tile i + 1 and the fold of tile i, in a fixed order
        Ops::template scores_fold<QG, TT>(next_buf, col, h, qf, nxt, cur, S, (unsigned)tis << 4);
      } else {
        Ops::template scores<QG>(next_buf, col, h, qf, nxt);
        absorb<QG, TT, false>(S, cur, tis, jb, jend, c);
        Ops::template interleave<QG, TT>();
      }
    } else if (do_cur && full) {
      absorb<QG, TT, false>(S, cur, tis, jb, jend, c);
    } else {
      if (do_next) Ops::template scores<QG>(next_buf, col, h, qf, nxt);
      if (do_cur) absorb<QG, TT, true>(S, cur, tis, jb, jend, c);
    }
    if (do_cur && (tis == kSegTiles - 1 || i + 1 == my_tiles))
      flush_segment<QG, TT>(S, L, (i - tis) * kTileB, h);
  };
  int i0 = 0;
  // (Only where it pays for its code size: the per-head bf16 gate with a
  // short list, i.e. top_k up to 5.)
  if constexpr (DMA && NBUF == 3 && std::is_same<Ops, GateOps<bf16, D>>::value && TT <= 6) {
    // Steady stretch: a segment of kSegTiles steps at a time with no
    // per-step conditions, while every wave of the workgroup has the
    // segment's tiles and the next one full, and the tiles the segment
    // loads exist (the counts are workgroup-uniform, so every wave takes
    // the same barriers). The general step takes the rest.
    const int n_full = min(min(wg_full[0], wg_full[1]), min(wg_full[2], wg_full[3]));
    auto steady = [&](int i, int k, f32x16(&cur)[QG], f32x16(&nxt)[QG]) {
      lds_dma_wait_n<Ops::NDMA>();
      __syncthreads();
      Ops::dma(a.kbar_hi + (kvb0 + (int64_t)(i + 3) * kTileB) * D, doff, lds_addr(buf(i + 3)), w);
      Ops::template scores_fold<QG, TT>(buf(i + 1), col, h, qf, nxt, cur, S, (unsigned)k << 4);
    };
    static_assert(kSegTiles == 8, "the steady stretch is unrolled over one segment");
    for (; i0 + kSegTiles + 1 <= n_full && i0 + kSegTiles + 2 < ntiles; i0 += kSegTiles) {
      steady(i0, 0, acc_a, acc_b);
      steady(i0 + 1, 1, acc_b, acc_a);
      steady(i0 + 2, 2, acc_a, acc_b);
      steady(i0 + 3, 3, acc_b, acc_a);
      steady(i0 + 4, 4, acc_a, acc_b);
      steady(i0 + 5, 5, acc_b, acc_a);
      steady(i0 + 6, 6, acc_a, acc_b);
      steady(i0 + 7, 7, acc_b, acc_a);
      flush_segment<QG, TT>(S, L, i0 * kTileB, h);
    }
  }
  for (int i = i0; i < ntiles; i += 2) {
    step(i, acc_a, acc_b);
    if (i + 1 < ntiles) step(i + 1, acc_b, acc_a);
  }
  if (!wave_on) return;

  const float kmax = fmaxf(fmaxf(wg_kmax[0], wg_kmax[1]), fmaxf(wg_kmax[2], wg_kmax[3]));
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int64_t t = tw + 32 * g + col;
    const bool qvalid = t < len;
    int sel[TT];
    if (scoring) {
      // Merge the two lane halves (keys are distinct, so both halves end
      // with the same list), then decode scores and block indices.
      double P[TT];
#pragma unroll
      for (int i = 0; i < TT; ++i) P[i] = shfl_xor32(L[g][i]);
#pragma unroll
      for (int i = 0; i < TT; ++i) insert_key(L[g], P[i]);
      float ls[TT];
      int lj[TT];
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        ls[i] = key_score(L[g][i]);
        lj[i] = key_block(L[g][i]);
        sel[i] = lj[i];
      }
      // ---- exactness check: is the cut between kept and dropped blocks
      // farther apart than twice the fast scores' rounding bound?
      // A shared gate's fp32 query sum adds at most (nq - 1) roundings of
      // 2^-24 per coordinate, covered by nq * 2^-22 against sum_h ||q_h||.
      const float gam = Ops::gamma() + (SHARED ? (float)nq * 2.3841858e-07f : 0.f);
      // Fast scores are bounded by ||q|| max ||kbar||; where that bound
      // leaves fp32 they may be infinite or NaN, which the lists drop, so
      // such a query is re-scanned in full (decided on the norms alone: the
      // build assumes no NaNs in comparisons).
      const bool beyond = qnorm[g] > 3.0e38f || kmax > 3.0e38f || qnorm[g] * kmax > 3.0e38f;
      const float eps = gam * qnorm[g] * kmax + 1e-30f;
      const bool amb = beyond || !(ls[m - 1] - ls[m] > 2.f * eps);
      const bool tracked = !beyond && (n_elig <= TT || ls[TT - 1] < ls[m - 1] - 2.f * eps);
      rescore_ambiguous<TQ, D, TT>(a, qrow0, len, nq, kvb0, tw + 32 * g, c, jend, amb && h == 0 && qvalid, tracked,
                                   lj, sel, lane, col, reinterpret_cast<double*>(tile) + w * D);
    }
    if (h == 0 && qvalid)
      for (int hq = 0; hq < nq; ++hq)
        write_row<TT>(a.block_idx + (qrow0 + hq * len + t) * a.top_k, sel, scoring, m, c, a.causal ? c + 1 : NB,
                      a.top_k);
  }
}

// Numbers every (query, kept past block) pair inside that block's query
// list: rank[q][slot] = position of q in the list of the slot's block.
// Workgroups of 1024 queries count their picks per block in LDS, reserve
// one contiguous range per block with a single global atomic, and add the
// range start to each pick's local position.
__global__ __launch_bounds__(256) void rank_kernel(GateArgs a) {
  extern __shared__ __align__(16) char smem[];
  int* bins = reinterpret_cast<int*>(smem);
  // Work item -> (sequence, query head, chunk of kRankQ queries).
  const int64_t item = blockIdx.x;
  const int64_t si = seq_find_u(a.sq, kSeqW1024, a.heads, item, a.block_size);
  const SeqAt sa = seq_at_u(a.sq, si, a.block_size);
  const int64_t per_head = (sa.len + kRankQ - 1) / kRankQ;
  const int64_t r_item = item - a.heads * seq_prefix_u(a.sq, si, kSeqW1024, a.block_size);
  const int64_t hq = r_item / per_head;
  const int64_t q0 = (r_item % per_head) * kRankQ;
  const int NB = (int)sa.nb;
  const bool lds_bins = a.max_nb <= kLdsBinsMax;  // LDS holds max_nb bins when this is true
  const int64_t row0 = sa.tok0 * a.heads + hq * sa.len;  // row of token 0 of this head
  const int slots = a.k_eff - 1;
  int32_t* cnt = a.count + sa.blk0 * a.heads + hq * NB;
  if (lds_bins)
    for (int i = threadIdx.x; i < NB; i += 256) bins[i] = 0;
  __syncthreads();
  for (int qq = threadIdx.x; qq < kRankQ; qq += 256) {
    const int64_t t = q0 + qq;
    if (t >= sa.len) break;
    const int c = (int)(t / a.block_size);
    const int32_t* row = a.block_idx + (row0 + t) * a.top_k;
    int32_t* rk = a.rank + (row0 + t) * (int64_t)slots;
    const int cap = past_cap(c, NB, a.causal, a.k_eff);
    int s = 0;
    for (int i = 0; i < a.top_k && s < cap; ++i) {
      const int j = row[i];
      if (j < 0) break;
      if (!routed_past_block(j, c, NB, a.causal)) continue;
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
    if (t >= sa.len) break;
    const int c = (int)(t / a.block_size);
    const int32_t* row = a.block_idx + (row0 + t) * a.top_k;
    int32_t* rk = a.rank + (row0 + t) * (int64_t)slots;
    const int cap = past_cap(c, NB, a.causal, a.k_eff);
    int s = 0;
    for (int i = 0; i < a.top_k && s < cap; ++i) {
      const int j = row[i];
      if (j < 0) break;
      if (!routed_past_block(j, c, NB, a.causal)) continue;
      rk[s++] += bins[j];
    }
  }
}

template <typename T, typename TQ, int D, int TT, bool SHARED, int QG = 1, int NBUF = 3>
static void gate_go(const GateArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(QG == 2 ? a.gate_wgs256 : a.gate_wgs));
  using Ops = typename pick_type<SHARED, GateOpsSplitQ<D>, GateOps<T, D>>::type;
  constexpr int NB = Ops::kDma ? NBUF : 2;
  const int lds = NB * Ops::TILE_BYTES;
  hipLaunchKernelGGL((gate_topk_kernel<T, TQ, D, TT, SHARED, QG, NB>), grid, dim3(256), lds, s, a);
}

template <typename T, typename TQ, int D, bool SHARED>
static void gate_pick(const GateArgs& a, hipStream_t s) {
  // The list tracks m + 2 or more blocks so that a rounding band at the
  // cut usually ends inside it.
  const int m = a.k_eff - 1;
  if constexpr (sizeof(T) == 2 && !SHARED) {
    if (m <= 4) {  // the per-head bf16 gate with short lists (see gate_waves)
      const bool two_groups = a.max_nb > kShortMaxBlocks;
      if (m <= 2) {
        if (two_groups) gate_go<T, TQ, D, 4, SHARED, 2>(a, s);
        else gate_go<T, TQ, D, 4, SHARED, 1, 2>(a, s);
      } else {
        if (two_groups) gate_go<T, TQ, D, 6, SHARED, 2>(a, s);
        else gate_go<T, TQ, D, 6, SHARED, 1, 2>(a, s);
      }
      return;
    }
  } else if constexpr (SHARED) {
    if (m <= 4) {
      if (m <= 2) gate_go<T, TQ, D, 4, SHARED, 1, 2>(a, s);
      else gate_go<T, TQ, D, 6, SHARED, 1, 2>(a, s);
      return;
    }
    if (m <= 2) {
      gate_go<T, TQ, D, 4, SHARED>(a, s);
      return;
    }
    if (m <= 4) {
      gate_go<T, TQ, D, 6, SHARED>(a, s);
      return;
    }
  } else {
    if (m <= 2) {
      gate_go<T, TQ, D, 4, SHARED>(a, s);
      return;
    }
    if (m <= 4) {
      gate_go<T, TQ, D, 6, SHARED>(a, s);
      return;
    }
  }
  if (m <= 8) gate_go<T, TQ, D, 10, SHARED>(a, s);
  else gate_go<T, TQ, D, kMaxSlots + 2, SHARED>(a, s);
}

// T: the stored dtype. A shared gate of a group of more than one head
// scores the fp32 sum of its queries, split into a bf16 pair.
template <typename T, int D>
static hipError_t gate_launch_t(const GateArgs& a, hipStream_t s) {
  {
    KernelTimer timer(s, "gate_topk");
    if (a.shared && a.group > 1) gate_pick<bf16, T, D, true>(a, s);
    else gate_pick<T, T, D, false>(a, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.k_eff < 2) return e;
  static_assert(kRankQ == 1024, "the sequence table counts rank workgroups of 1024 queries");
  const int rank_lds = a.max_nb <= kLdsBinsMax ? (int)a.max_nb * 4 : 0;
  {
    KernelTimer timer(s, "rank");
    hipLaunchKernelGGL(rank_kernel, dim3((unsigned)a.rank_wgs), dim3(256), rank_lds, s, a);
  }
  return hipGetLastError();
}

// Ranks in a fixed order (for sums over a block's list that must not
// depend on scheduling): chunk_count counts each chunk's picks per block,
// chunk_scan turns them into per-chunk bases (and the block totals in
// count), and rank_ordered numbers the picks of a chunk in the order
// (64-query group, column of block_idx, lane) with wave ballots: lanes
// with the same block in one column get consecutive ranks by lane.
__global__ __launch_bounds__(256) void chunk_count_kernel(GateArgs a, int32_t* cc, int64_t nchunk, int qchunk) {
  extern __shared__ __align__(16) char smem[];
  int* bins = reinterpret_cast<int*>(smem);
  const int NB = (int)a.n_blocks;
  const int64_t bh = blockIdx.x / nchunk, ch = blockIdx.x % nchunk;
  for (int i = threadIdx.x; i < NB; i += 256) bins[i] = 0;
  __syncthreads();
  for (int qq = threadIdx.x; qq < qchunk; qq += 256) {
    const int64_t t = ch * qchunk + qq;
    if (t >= a.seq_len) break;
    const int c = (int)(t / a.block_size);
    const int32_t* row = a.block_idx + (bh * a.seq_len + t) * a.top_k;
    const int cap = past_cap(c, NB, a.causal, a.k_eff);
    int s = 0;
    for (int i = 0; i < a.top_k && s < cap; ++i) {
      const int j = row[i];
      if (j < 0) break;
      if (!routed_past_block(j, c, NB, a.causal)) continue;
      atomicAdd(bins + j, 1);
      ++s;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NB; i += 256) cc[(bh * nchunk + ch) * NB + i] = bins[i];
}

__global__ __launch_bounds__(256) void chunk_scan_kernel(GateArgs a, int32_t* cc, int64_t nchunk) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int NB = (int)a.n_blocks;
  if (id >= a.bh * NB) return;
  const int64_t bh = id / NB, j = id % NB;
  int32_t* p = cc + bh * nchunk * NB + j;  // chunk ch at p[ch * NB]
  int32_t run = 0;
  int64_t ch = 0;
  // Eight counts requested before the first of their bases is stored.
  for (; ch + 8 <= nchunk; ch += 8) {
    int32_t n[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) n[u] = p[(ch + u) * NB];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      p[(ch + u) * NB] = run;
      run += n[u];
    }
  }
  for (; ch < nchunk; ++ch) {
    const int32_t n = p[ch * NB];
    p[ch * NB] = run;
    run += n;
  }
  a.count[id] = run;
}

__global__ __launch_bounds__(64) void rank_ordered_kernel(GateArgs a, const int32_t* cc, int64_t nchunk, int qchunk) {
  extern __shared__ __align__(16) char smem[];
  int* bins = reinterpret_cast<int*>(smem);
  const int NB = (int)a.n_blocks;
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x / nchunk, ch = blockIdx.x % nchunk;
  const int slots = a.k_eff - 1;
  for (int i = lane; i < NB; i += 64) bins[i] = cc[(bh * nchunk + ch) * NB + i];
  __syncthreads();
  for (int g = 0; g < qchunk; g += 64) {
    const int64_t t = ch * qchunk + g + lane;
    const bool on = t < a.seq_len;
    const int c = on ? (int)(t / a.block_size) : -1;
    const int32_t* row = a.block_idx + (bh * a.seq_len + (on ? t : 0)) * a.top_k;
    int32_t* rk = a.rank + (bh * a.seq_len + (on ? t : 0)) * (int64_t)slots;
    int s = 0;          // this lane's past-block index so far
    bool done = !on;    // a -1 ends the row
    for (int i = 0; i < a.top_k; ++i) {
      int j = done ? -1 : row[i];
      if (j < 0) done = true;
      const bool pick = !done && s < past_cap(c, NB, a.causal, a.k_eff) && routed_past_block(j, c, NB, a.causal);
      uint64_t todo = __builtin_amdgcn_ballot_w64(pick);
      while (todo) {
        const int leader = __builtin_ctzll(todo);
        const int jl = __builtin_amdgcn_readlane(j, leader);
        const uint64_t same = __builtin_amdgcn_ballot_w64(pick && j == jl);
        const int base = bins[jl];
        if (pick && j == jl) rk[s] = base + __builtin_popcountll(same & ((1ull << lane) - 1));
        __syncthreads();  // every lane has read bins[jl] before it moves
        if (lane == leader) bins[jl] = base + __builtin_popcountll(same);
        __syncthreads();
        todo &= ~same;
      }
      if (pick) ++s;
    }
  }
}

hipError_t launch_rank(const GateArgs& a, hipStream_t s, int32_t* chunk_counts) {
  if (a.k_eff < 2) return hipSuccess;
  const int qchunk = (int)rank_chunk(a.seq_len);
  const int64_t nchunk = (a.seq_len + qchunk - 1) / qchunk;
  const int lds = (int)a.n_blocks * 4;
  if (lds > 65536) return hipErrorInvalidValue;
  KernelTimer timer(s, "rank_ordered");
  hipLaunchKernelGGL(chunk_count_kernel, dim3((unsigned)(a.bh * nchunk)), dim3(256), lds, s, a, chunk_counts, nchunk,
                     qchunk);
  hipLaunchKernelGGL(chunk_scan_kernel, dim3((unsigned)((a.bh * a.n_blocks + 255) / 256)), dim3(256), 0, s, a,
                     chunk_counts, nchunk);
  hipLaunchKernelGGL(rank_ordered_kernel, dim3((unsigned)(a.bh * nchunk)), dim3(64), lds, s, a, chunk_counts, nchunk,
                     qchunk);
  return hipGetLastError();
}

hipError_t launch_gate(const GateArgs& a, hipStream_t s) {
  if (a.bf16_in) return a.head_dim == 128 ? gate_launch_t<bf16, 128>(a, s) : gate_launch_t<bf16, 64>(a, s);
  return a.head_dim == 128 ? gate_launch_t<float, 128>(a, s) : gate_launch_t<float, 64>(a, s);
}

}  // namespace moba
