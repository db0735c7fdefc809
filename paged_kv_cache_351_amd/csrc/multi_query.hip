// Multi-query paged attention for gfx950 (CDNA4): several query tokens per
// sequence, each attending causally to the sequence's cached tokens -- the
// attention of chunked prefill (a long prompt processed in pieces) and of
// speculative verification (several drafted tokens scored at once), both of
// which the pages pair with PagedAttention ("PagedAttention：分页注意力——推理引擎的显存革命",
// section "2026年最新进展").  Sequence s owns query rows q_start[s] ..
// q_start[s+1]-1, its last n_s tokens (already in the cache); query i sits at
// position p = L_s - n_s + i and attends to tokens 0..p:
//     out[row, h] = softmax_t<=p(scale * q[row, h] . K_s[t]) V_s[t],
// K/V fetched through the block table ("LLM 注意力与计算内核精读笔记 · 05
// PagedAttention 与 KV 显存管理", §3, §4), the softmax merged tile by tile with a
// running maximum and sum (same page, §4).
//
// Work decomposition
//   A workgroup (4 waves) owns one (sequence, KV head, query block, context
//   partition).  A query block is 16 rows (the split variant below), 64 rows (16
//   per wave) or 128 rows (32 per wave, two row blocks of 16): consecutive query
//   tokens times the g query heads of the KV head's group, row = token * g + head.
//   The context up to the block's last query position is cut into `parts` equal
//   partitions of whole tiles.  With one partition the workgroup writes the output;
//   otherwise it leaves (m, l, acc) per row and a second kernel merges the
//   partitions in order.  Workgroups are numbered so that every query block and
//   partition of one (sequence, KV head) runs on the same XCD (workgroup id mod 8),
//   where they share its L2, and consecutive (sequence, KV head) units run on
//   different XCDs.
//
// Per tile of 32 tokens
//   The tile's K and V rows (16 bytes per load, token -> block through the table,
//   table entries one step earlier than the rows) are loaded ahead into registers
//   and stored to LDS as [token][head_dim] rows.  Then each wave, on the matrix
//   cores:
//     S^T = K Q^T   v_mfma_f32_16x16x32_{bf16,f16} (16x16x4_f32 for fp32): A = K
//                   rows of one 16-token half, B = the wave's 16 query rows, both
//                   cut into the same head_dim chunks; lane (grp, col) gets the
//                   scores of tokens 16 h + 4 grp + i, i = 0..3, for row col.
//     online softmax per row: exponentials in base 2 against a reference maximum
//                   that moves only when a tile exceeds it by 2^8.
//     O^T += V^T P^T with A = V^T (16 head_dim rows x 32 slots) and B = P^T:
//                   slot 8 grp + 4 h + i stands for token 16 h + 4 grp + i, so
//                   lane (grp, col) holds P for slots 8 grp .. 8 grp + 7, exactly
//                   the tokens whose scores it computed, and the scores never move
//                   between lanes.  The LDS transpose read (ds_read_b64_tr_b16)
//                   turns the [token][head_dim] V rows into the A fragments.
//   Shared tiles of 16-bit types run a pipelined loop: tile k + 1's scores are
//   computed while tile k's weights are formed, in explicitly interleaved chunks of
//   matrix and vector instructions (see run_pipelined).
//   P enters the second product in a 16-bit type.  fp16 data: P rounded to fp16
//   (11 significant bits).  bf16 data with shared tiles (prefill-sized blocks): V
//   is staged in LDS as fp16 (exact for |v| < 2^16) and P rounded to fp16, one
//   product; a V value beyond fp16's range becomes inf, the workgroup's result
//   comes out non-finite, and the workgroup runs its tiles again with bf16 V and
//   the two-term P below (so every finite input is handled, the common case at one
//   product per tile instead of two).  bf16 data in the split variant: P split into
//   two bf16 terms (about 16 significant bits) fed to two products.  fp32 stays
//   fp32.  The running sum adds the weights used (in the pipelined loop as a matrix
//   product of P with a block of ones; elsewhere, for two-term bf16, the fp32
//   values, within 2^-16 of the two terms), so the output is a weighted mean with
//   the weights used.  Scores stay raw until the exponent, p = 2^(s * |scale|
//   log2 e - m) in one fused multiply-add (a negative scale is folded into q's
//   signs).  Masked tokens get -inf, i.e. weight 0; running maxima start at -1e30
//   so no row ever forms inf - inf.
#include <type_traits>

#include "multi_query.h"

namespace pagedkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 32;   // tokens per K/V tile
constexpr float kNegBig = -1.0e30f;
constexpr float kLazyMax = 8.0f;   // a row's reference maximum may trail by up to 2^8

template <int DT, int D>
struct Shape {
  static constexpr int EB = DT == kF32 ? 4 : 2;   // bytes per element
  static constexpr int ROWB = D * EB;             // bytes per K/V row
  static constexpr int CR = ROWB / 16;            // 16-byte chunks per row
  static constexpr int NKC = CR / 4;              // chunks per lane of one row (4 lane groups)
  static constexpr int KSTRIDE = ROWB + 16;       // LDS bytes per K row, padded
  static constexpr int VSTRIDE = ROWB + 32;       // LDS bytes per V row: four rows' 32-byte
                                                  // pieces fall in distinct banks
  static constexpr int KBYTES = kTile * KSTRIDE;
  static constexpr int VBYTES = kTile * VSTRIDE;
  static constexpr int LDS = KBYTES + VBYTES;
  static constexpr int KLOADS = kTile * CR / 256;         // tokens per thread per tile
  static constexpr int NJ = D / 16;                       // 16-row head_dim blocks of O^T
  static_assert(KLOADS >= 1 && kTile * CR % 256 == 0, "tile does not split over 256 lanes");
};

// Chunk (16 bytes) of a row that lane group grp feeds to the matrix cores in step c.
template <int DT, int D>
__device__ __forceinline__ int chunk_of(int c, int grp) {
  if constexpr (DT == kF32) return grp * Shape<DT, D>::NKC + c;  // 4 floats, one per MFMA
  else return 4 * c + grp;                                        // 8 halves, one MFMA
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Four 16-bit elements through the LDS transpose read (ds_read_b64_tr_b16).  In each
// group of 16 lanes, lane i names 8 bytes (elements M[i][0..3]); lane j receives
// M[4q + j/4][j%4] for q = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum over lanes i, i ^ 16, i ^ 32 and i ^ 48 with the gfx950 row swaps (no trip
// through LDS): swapping a value with a copy of itself leaves one lane of each pair
// in each result, so the maximum of the two results is the pair's maximum.
__device__ __forceinline__ float max_over_groups(float x) {
  // (left-leaning chains, so that each step is one v_max3 and the swapped values are not
  // first passed through a canonicalising maximum of their own)
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(fmaxf(x, __uint_as_float(a[0])), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(fmaxf(x, __uint_as_float(b[0])), __uint_as_float(b[1]));
}

// The same with the IEEE maximum (NaN-propagating, gfx950 v_maximum3_f32): no canonicalising
// instruction before each maximum.  Used where a NaN score makes the row's result non-finite
// either way.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max_over_groups_nan(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float vmax8(const f32x4& a, const f32x4& b) {
  return vmax(vmax(vmax(vmax(vmax(vmax(vmax(a[0], a[1]), a[2]), a[3]), b[0]), b[1]), b[2]), b[3]);
}

template <int DT>
__device__ __forceinline__ uint16_t to_store(float x) {
  if constexpr (DT == kBF16) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Two values rounded to the storage type in one packed conversion, the first in the
// low half.
template <int DT>
__device__ __forceinline__ uint32_t to_store2(float a, float b) {
  if constexpr (DT == kBF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
  }
}

template <int DT>
__device__ __forceinline__ float from_store(uint16_t x) {
  if constexpr (DT == kBF16) return __uint_as_float((uint32_t)x << 16);
  else return (float)__builtin_bit_cast(_Float16, x);
}

// Store 4 consecutive output elements.
template <int DT>
__device__ __forceinline__ void store4(void* dst, f32x4 v) {
  if constexpr (DT == kF32) {
    *reinterpret_cast<f32x4*>(dst) = v;
  } else {
    const uint32_t a = (uint32_t)to_store<DT>(v[0]) | ((uint32_t)to_store<DT>(v[1]) << 16);
    const uint32_t b = (uint32_t)to_store<DT>(v[2]) | ((uint32_t)to_store<DT>(v[3]) << 16);
    *reinterpret_cast<u32x2*>(dst) = u32x2{a, b};
  }
}

// Decode the workgroup's item: XCD-major numbering, then (s, kv, qb, part).
struct Item {
  int s, kv, qb, part;
};

// Decode the workgroup's item.  The (sequence, KV head) units are dealt to the 8
// XCDs in turn (workgroup b runs on XCD b mod 8), unit u to XCD u mod 8, and every
// query block and partition of a unit stays on its XCD, where they share its L2: the
// XCDs get equal shares of every sequence's KV heads rather than whole sequences.
// Each XCD takes its units in order, a unit's last query block (the most context)
// first; with an ordering the units' sequences (groups) come longest first, so that
// the last items to start are the shortest.  The grid is 8 * ceil(units / 8) *
// (query blocks * partitions) workgroups.
__device__ __forceinline__ bool item_of(const MultiQueryParams& p, Item& it) {
  const long long b = blockIdx.x;
  const long long ipu = (long long)p.qblocks * p.parts;   // items per unit
  const long long j = b / 8;
  const long long u = (j / ipu) * 8 + b % 8;
  if (u >= (long long)p.num_seqs * p.num_kv_heads) return false;
  const long long r = j % ipu;
  it.part = (int)(r % p.parts);
  it.qb = p.qblocks - 1 - (int)(r / p.parts);
  it.kv = (int)(u % p.num_kv_heads);
  int s = (int)(u / p.num_kv_heads);
  if (p.order) {
    s = p.order[s];
    if (s < 0 || s >= p.num_seqs) return false;
  }
  it.s = s;
  return true;
}

// Longest-first ordering of the items' sequences (multi-query) or groups (shared
// prefix), one workgroup: a counting sort on the number of 32-token tiles (capped),
// written to order_out.  Equal keys may come out in any order; each item's result
// does not depend on which workgroup computes it.
constexpr int kOrderBuckets = 4096;

template <bool SHARED>
__global__ __launch_bounds__(1024) void item_order_kernel(MultiQueryParams p) {
  __shared__ int hist[kOrderBuckets];
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  auto clamp_len = [&](int x) { return x < 0 ? 0 : (x > p.max_seq_len ? p.max_seq_len : x); };
  auto bucket = [&](int s) {
    int tiles;
    if constexpr (!SHARED) {
      tiles = (clamp_len(p.seq_lens[s]) + kTile - 1) / kTile;
    } else {
      const int a = p.q_start[s];
      int n = p.q_start[s + 1] - a;
      n = n < 0 ? 0 : (n > p.max_q_len ? p.max_q_len : n);
      if (a < 0 || a + n > p.total_q) n = 0;
      int lmin = 0x7fffffff;
      for (int i = 0; i < n; ++i) lmin = min(lmin, clamp_len(p.seq_lens[a + i]));
      const int P = n > 0 ? min(clamp_len(p.prefix_lens[s]), lmin) : 0;
      tiles = (P + kTile - 1) / kTile;
      for (int i = 0; i < n && tiles < kOrderBuckets; ++i)
        tiles += (clamp_len(p.seq_lens[a + i]) - P + kTile - 1) / kTile;
    }
    return kOrderBuckets - 1 - min(tiles, kOrderBuckets - 1);  // ascending bucket = descending work
  };
  for (int i = tid; i < kOrderBuckets; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int s = tid; s < p.num_seqs; s += 1024) atomicAdd(&hist[bucket(s)], 1);
  __syncthreads();
  // exclusive prefix sum of the histogram: thread t owns buckets 4t .. 4t+3
  const int h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2], h3 = hist[4 * tid + 3];
  const int mine = h0 + h1 + h2 + h3;
  part[tid] = mine;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const int base = part[tid] - mine;
  hist[4 * tid] = base;
  hist[4 * tid + 1] = base + h0;
  hist[4 * tid + 2] = base + h0 + h1;
  hist[4 * tid + 3] = base + h0 + h1 + h2;
  __syncthreads();
  for (int s = tid; s < p.num_seqs; s += 1024) p.order_out[atomicAdd(&hist[bucket(s)], 1)] = s;
}

// Where the 32 tokens of one tile come from: tokens base .. base + count - 1 of
// the sequence whose block table is `table`; slots past `count` are masked (and
// read as a copy of the last valid token).  owner >= 0: only the rows of that
// member may see the tile (a member's private tail in a shared-prefix group).
struct TileMap {
  const int32_t* table;
  int base, count, owner;
};

// SPLIT = false: the four waves own 16 RB rows each of a 64 RB-row query block
// and share every K/V tile through LDS (prefill-sized blocks); with RB = 2 every
// K/V fragment read from LDS feeds two 16-row products, and registers are capped
// for two waves per SIMD (16-bit types) so that two workgroups share a CU across
// the barriers.
// SPLIT = true (16-bit types, at most 16 rows per block, RB = 1): the four waves
// work on the same 16 rows and take every fourth tile of the partition each, K
// straight from HBM into registers in the matrix-core layout and V through a
// wave-private LDS region, with no workgroup barrier in the loop; their four
// partial results are merged through LDS at the end.
// SHARED (split only): the item is a group of sequences whose first tokens sit in
// the same blocks; rows are (member, head), and the tiles are the shared prefix
// (read once, seen by every member) followed by each member's own tail (seen by
// that member only), each padded to whole tiles.
template <int DT, int D, bool SPLIT, bool SHARED, int RB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RB == 2 && DT != kF32 ? 2 : 1)))
void multi_query_kernel(MultiQueryParams p) {
  using S = Shape<DT, D>;
  constexpr int EB = S::EB, CR = S::CR, NKC = S::NKC, NJ = S::NJ;
  constexpr int VREG = S::VBYTES;                          // one V tile
  // shared tiles of 16-bit types run the pipelined loop below on three LDS buffers; fp32
  // runs the plain loop on two
  constexpr bool PIPE = !SPLIT && DT != kF32;
  constexpr int LDS_BYTES = SPLIT ? 4 * VREG : (PIPE ? 3 : 2) * S::LDS;
  static_assert(!SPLIT || (DT != kF32 && 4 * 16 * (D + 2) * 4 <= LDS_BYTES), "split merge space");
  static_assert(SPLIT || !SHARED, "shared-prefix groups use the split variant");
  static_assert(RB == 1 || (RB == 2 && !SPLIT), "two row blocks only with shared tiles");
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  // bf16 with shared tiles: V is staged in LDS as fp16 and P.V runs as one fp16 product
  // (see softmax_pv); a workgroup whose result comes out non-finite (a V value beyond
  // fp16's range, or non-finite input) runs its tiles again with bf16 V (see the end of
  // the tile loop)
  constexpr bool PVH = DT == kBF16 && !SPLIT;
  __shared__ uint32_t redo_flag[4];

  Item it;
  if (!item_of(p, it)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int g = p.group, Hq = p.num_heads, Hkv = p.num_kv_heads;
  char* const ldsV = lds + wave * VREG;   // the split variant's V region

  // The item's rows: query tokens qa + tok0 .. qa + tok1 - 1 of one sequence (multi-query),
  // or member sequences qa + tok0 .. qa + tok1 - 1 of one group (shared prefix), g heads
  // each.  Everything read from the index arrays is clamped so no access leaves them.
  const int qa = p.q_start[it.s];
  int n = p.q_start[it.s + 1] - qa;
  n = n < 0 ? 0 : (n > p.max_q_len ? p.max_q_len : n);
  if (qa < 0 || qa + n > p.total_q) n = 0;
  const int tok0 = it.qb * p.tq;
  if (tok0 >= n) return;
  const int tok1 = min(n, tok0 + p.tq);
  auto clamp_len = [&](int x) { return x < 0 ? 0 : (x > p.max_seq_len ? p.max_seq_len : x); };

  // this lane's rows: row col of each of the wave's RB blocks of 16
  int qtok[RB], qh[RB];
  bool row_ok[RB];
  size_t out_row[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rloc = SPLIT ? col : (wave * RB + b) * 16 + col;
    qtok[b] = tok0 + rloc / g;
    qh[b] = rloc % g;
    row_ok[b] = rloc < p.tq * g && qtok[b] < tok1;
    out_row[b] = (size_t)(qa + qtok[b]) * Hq + (size_t)it.kv * g + qh[b];
  }

  int L = 0, pos_lo = 0, t_end = 0;                // multi-query
  int pos[RB];                                      // each row's causal limit (inclusive)
  int P = 0, VP = 0, m_off = 0, m_tail = 0;        // shared prefix: lane i < tok1 - tok0 = member i
  const int32_t* tables = p.block_tables;
  const int32_t* seq_table = nullptr;
  if constexpr (!SHARED) {
    L = clamp_len(p.seq_lens[it.s]);
    const int pos_hi = L - n + tok1 - 1;           // last query position of the block
    pos_lo = L - n + tok0;                         // first query position of the block
#pragma unroll
    for (int b = 0; b < RB; ++b) pos[b] = L - n + qtok[b];
    t_end = min(L, pos_hi + 1);
    seq_table = tables + (size_t)it.s * p.max_blocks_per_seq;
  } else {
    const int cnt = tok1 - tok0;
    const int mine = lane < cnt ? clamp_len(p.seq_lens[qa + tok0 + lane]) : 0x7fffffff;
    // member data lives in lanes 0..15; reductions run inside that 16-lane row and
    // their results are broadcast from it, so every lane agrees on P and t_end
    int lmin = mine;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) lmin = min(lmin, __shfl_xor(lmin, o));
    lmin = __shfl(lmin, 0);
    P = min(clamp_len(p.prefix_lens[it.s]), lmin);  // a prefix longer than a member is cut
    VP = (P + kTile - 1) / kTile * kTile;
    m_tail = lane < cnt ? mine - P : 0;
    const int padded = (m_tail + kTile - 1) / kTile * kTile;
    int incl = padded;                             // prefix sum over lanes 0..15
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int v = __shfl_up(incl, o, 16);
      if ((lane & 15) >= o) incl += v;
    }
    m_off = incl - padded;
    t_end = VP + __shfl(incl, 15);
    seq_table = tables + (size_t)(qa + tok0) * p.max_blocks_per_seq;  // the group's first member
#pragma unroll
    for (int b = 0; b < RB; ++b) pos[b] = 0;
  }
  // with several partitions, the item's own range is cut into equal whole tiles
  int t_begin = 0;
  if (p.parts > 1) {
    const int plen = ((t_end + p.parts - 1) / p.parts + kTile - 1) / kTile * kTile;
    t_begin = it.part * plen;
    t_end = min(t_end, t_begin + plen);
  }

  // Source of the tile starting at t0 (uniform over the workgroup).
  auto tile_map = [&](int t0) -> TileMap {
    TileMap mp;
    if constexpr (!SHARED) {
      mp = TileMap{seq_table, t0, min(kTile, t_end - t0), -1};
    } else {
      if (t0 < VP) {
        mp = TileMap{seq_table, t0, min(kTile, P - t0), -1};
      } else {
        const int rel = t0 - VP;
        const unsigned long long below = __ballot(lane < tok1 - tok0 && m_off <= rel);
        const int owner = __popcll(below & 0xffffull) - 1;
        const int off = __shfl(m_off, owner), tail = __shfl(m_tail, owner);
        mp = TileMap{tables + (size_t)(qa + tok0 + owner) * p.max_blocks_per_seq, P + rel - off,
                     min(kTile, tail - (rel - off)), owner};
      }
    }
    return mp;
  };

  // query fragments: the same chunks of the row as the K fragments.  A negative scale is
  // folded into q (every sign flipped, which negates each score exactly), so the scores
  // are scaled by |scale| log2(e) > 0 and the maximum of the raw scores is the maximum of
  // the scaled ones.
  const bool neg_scale = p.scale_log2e < 0.f;
  const uint32_t qsign = neg_scale ? (DT == kF32 ? 0x80000000u : 0x80008000u) : 0u;
  u32x4 qf[RB][NKC];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      qf[b][c] = u32x4{0u, 0u, 0u, 0u};
      if (row_ok[b])
        qf[b][c] = *reinterpret_cast<const u32x4*>((const char*)p.q + out_row[b] * S::ROWB +
                                                   chunk_of<DT, D>(c, grp) * 16) ^ qsign;
    }

  f32x4 acc[RB][NJ];
  float m[RB], l[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[b] = kNegBig;
    l[b] = 0.f;
  }

  const int B = p.block_size;
  const size_t kv_off = (size_t)it.kv * S::ROWB;
  const size_t slot_bytes = (size_t)Hkv * S::ROWB;
  // Each lane loads the K and V rows of NT tokens of a tile (the same tokens for both):
  // the split variant tokens col and col + 16, NKC chunks each, straight in the matrix
  // core layout of K; the shared-tile variant tokens tid / CR + (256 / CR) k, chunk
  // tid % CR.  Tokens past a tile's count read its last valid token, so nothing outside
  // a sequence is read.  A token's block-table entry is fetched one step before its
  // rows, so that waiting for it never waits for the rows in flight.
  // (the pipelined loop: eight lanes per token, CR / 8 chunks each, so that a lane looks up
  // one token per tile)
  static_assert(!PIPE || CR % 8 == 0, "eight lanes per row");
  constexpr int NT = SPLIT ? 2 : (PIPE ? 1 : S::KLOADS);      // tokens per lane per tile
  constexpr int CPT = SPLIT ? NKC : (PIPE ? CR / 8 : 1);      // 16-byte chunks per token
  constexpr int KL = NT * CPT;
  auto my_tok = [&](int k) { return SPLIT ? col + 16 * k : (PIPE ? tid >> 3 : tid / CR + (256 / CR) * k); };
  auto my_chunk = [&](int c) { return SPLIT ? chunk_of<DT, D>(c, grp) : (PIPE ? (tid & 7) + 8 * c : tid % CR); };
  const float inv_b = p.inv_block_size;
  const int log2_b = p.log2_block_size;
  // block-table entries (tb) and in-block offsets (to) of this lane's tokens of a tile
  auto fetch_table = [&](int (&tb)[NT], int (&to)[NT], const TileMap& mp) {
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const int t = mp.base + min(my_tok(k), mp.count - 1);
      int j, o;
      if (log2_b >= 0) {   // a power-of-two block size (uniform): a shift and a mask
        j = t >> log2_b;
        o = t & (B - 1);
      } else {
        // t / B without a branch or an integer division: t < 2^24 is exact in float,
        // the product is off by at most one, and one correction each way fixes it
        j = (int)((float)t * inv_b);
        o = t - j * B;
        j = o < 0 ? j - 1 : (o >= B ? j + 1 : j);
        o = o < 0 ? o + B : (o >= B ? o - B : o);
      }
      to[k] = o;
      tb[k] = mp.table[j];
    }
  };
  u32x4 kr[2][KL], vr[2][KL];
  // V rows go to LDS as they are ([token][head_dim], padded rows); the shared-tile
  // variant stores K the same way
  // Stage a tile's K/V rows in LDS.  For PVH, V goes in as fp16 unless SAFE: bf16 ->
  // fp16 is exact for |v| < 2^16 (8 significant bits fit in 11; below 2^-17 the fp16
  // spacing 2^-24 bounds the change); a larger value becomes inf and makes the result
  // non-finite, which sends the workgroup through its tiles again with SAFE set.
  auto store_kv = [&](auto safe_c, const u32x4 (&xk)[KL], const u32x4 (&xv)[KL], char* kb, char* vb) {
    constexpr bool SAFE = decltype(safe_c)::value;
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        u32x4 v = xv[k * CPT + c];
        if constexpr (PVH && !SAFE) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] = to_store2<kF16>(__uint_as_float(v[i] << 16), __uint_as_float(v[i] & 0xffff0000u));
        }
        *reinterpret_cast<u32x4*>(vb + my_tok(k) * S::VSTRIDE + my_chunk(c) * 16) = v;
        if constexpr (!SPLIT)
          *reinterpret_cast<u32x4*>(kb + my_tok(k) * S::KSTRIDE + my_chunk(c) * 16) = xk[k * CPT + c];
      }
  };

  const float sl2 = neg_scale ? -p.scale_log2e : p.scale_log2e;   // >= 0
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;

  // S^T = K Q^T for the two 16-token halves and every row block; a(h, c) gives the
  // K fragment of half h, step c
  f32x4 sc[RB][2];
  auto qk_to = [&](f32x4 (&sc)[RB][2], auto a) {
#pragma unroll
    for (int b = 0; b < RB; ++b) sc[b][0] = sc[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        const u32x4 kf = a(h, c);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          if constexpr (DT == kBF16) {
            sc[b][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf),
                                                               __builtin_bit_cast(bf16x8, qf[b][c]), sc[b][h], 0, 0, 0);
          } else if constexpr (DT == kF16) {
            sc[b][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kf),
                                                              __builtin_bit_cast(f16x8, qf[b][c]), sc[b][h], 0, 0, 0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sc[b][h] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf[e]), __uint_as_float(qf[b][c][e]),
                                                              sc[b][h], 0, 0, 0);
          }
        }
      }
  };
  auto qk = [&](auto a) { qk_to(sc, a); };

  // Online softmax of tile t0 (scores in sc) and O^T += V^T P^T from the V tile at vb
  // in LDS (fp16 for PVH unless SAFE; see store_kv).
  auto softmax_pv = [&](auto safe_c, int t0, const TileMap& mp, const char* vb) {
    constexpr bool SAFE = decltype(safe_c)::value;
    // tile token 16 h + 4 grp + i of row col; full tiles that every row may see in
    // full need no mask.  The raw scores are kept (masked ones -inf) and scaled inside
    // the exponent's fused multiply-add: p = 2^(s sl2 - m).
    float pr[RB][8], alpha[RB], tmax[RB], sv[RB][8];
    const bool whole = mp.count == kTile && (SHARED ? mp.owner < 0 : t0 + kTile - 1 <= pos_lo);
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (whole) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[b][4 * h + i] = sc[b][h][i];
      } else {
        const bool row_sees = !SHARED || mp.owner < 0 || mp.owner == qtok[b] - tok0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int u = 16 * h + 4 * grp + i;
            const bool ok = SHARED ? (row_sees && u < mp.count) : (u < mp.count && t0 + u <= pos[b]);
            sv[b][4 * h + i] = ok ? sc[b][h][i] : -__builtin_inff();
          }
      }
      // a left-leaning chain: the compiler makes it one maximum and three v_max3
      float mx = fmaxf(fmaxf(fmaxf(sv[b][0], sv[b][1]), sv[b][2]), sv[b][3]);
      mx = fmaxf(fmaxf(fmaxf(fmaxf(mx, sv[b][4]), sv[b][5]), sv[b][6]), sv[b][7]);
      mx = max_over_groups(mx);
      // a row with no visible token here has mx = -inf; with a zero scale that product is
      // NaN, which fmaxf drops
      tmax[b] = fmaxf(m[b], mx * sl2);
    }
    // The reference maximum of a row moves only when the tile's maximum exceeds it by
    // more than kLazyMax (base 2), for every row of the wave at once; otherwise the
    // weights are taken against the old reference, so they stay below 2^kLazyMax and
    // the accumulators need no rescaling.  Any reference gives the same normalised
    // result: acc and l are always relative to the same m.
    bool grow = false;
#pragma unroll
    for (int b = 0; b < RB; ++b) grow = grow || tmax[b] > m[b] + kLazyMax;
    const bool rescale = __any(grow);
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const float mn = rescale ? tmax[b] : m[b];
      alpha[b] = rescale ? fast_exp2(m[b] - mn) : 1.0f;
      m[b] = mn;
#pragma unroll
      for (int u = 0; u < 8; ++u) pr[b][u] = fast_exp2(fmaf(sv[b][u], sl2, -mn));
    }
    // a masked score (-inf) gives exactly 0 as long as sl2 > 0; with a zero scale
    // -inf * 0 is NaN, so those weights are cleared here (a uniform, rare branch)
    if (sl2 == 0.f && !whole) {
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int u = 0; u < 8; ++u) pr[b][u] = sv[b][u] == -__builtin_inff() ? 0.f : pr[b][u];
    }
    if (rescale) {
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[b][j] *= alpha[b];
    }

    // fp32 products: product u takes slot 8 grp + u, i.e. tile token 16 (u / 4) + 4 grp +
    // u % 4, at head_dim 16 j + col
    auto pv_f32 = [&]() {
#pragma unroll
      for (int b = 0; b < RB; ++b)
        l[b] = l[b] * alpha[b] + (((pr[b][0] + pr[b][1]) + (pr[b][2] + pr[b][3])) +
                                  ((pr[b][4] + pr[b][5]) + (pr[b][6] + pr[b][7])));
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          a[u] = *reinterpret_cast<const float*>(vb + (16 * (u >> 2) + 4 * grp + (u & 3)) * S::VSTRIDE +
                                                 (16 * j + col) * 4);
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], pr[b][u], acc[b][j], 0, 0, 0);
      }
    };
    // A = V^T for head_dim 16 j .. 16 j + 15 through two transpose reads: slots
    // 8 grp + 4 h + q hold tile tokens 16 h + 4 grp + q, and lane (grp, col) names the
    // row 16 h + 4 grp + col / 4 at head_dim 16 j + 4 (col % 4)
    const char* vbase = vb + (4 * grp + (col >> 2)) * S::VSTRIDE + (4 * (col & 3)) * 2;
    auto vfrag = [&](int j) {
      const s16x4 a0 = lds_read_tr16(vbase + 32 * j);
      const s16x4 a1 = lds_read_tr16(vbase + 16 * S::VSTRIDE + 32 * j);
      return __builtin_bit_cast(u32x4, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // P rounded once to fp16 (11 significant bits; the weights are below 2^8, so no
    // overflow), V in fp16 (its own type, or bf16 widened exactly): one product.  The
    // running sum adds the rounded weights, two at a time.
    auto pv_f16 = [&]() {
      const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
      u32x4 pb[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        uint32_t pw[4];
        float ps = l[b] * alpha[b];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          pw[u] = to_store2<kF16>(pr[b][2 * u], pr[b][2 * u + 1]);
          ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw[u]), one2, ps, false);
        }
        l[b] = ps;
        pb[b] = u32x4{pw[0], pw[1], pw[2], pw[3]};
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4 a = vfrag(j);
#pragma unroll
        for (int b = 0; b < RB; ++b)
          acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                             __builtin_bit_cast(f16x8, pb[b]), acc[b][j], 0, 0, 0);
      }
    };
    // bf16 P split into two bf16 terms fed to two products with the same bf16 V fragment
    // (bf16 alone keeps 8 significant bits): the high term is P cut to its top 16 bits,
    // which leaves an exact fp32 remainder, and the low term is that remainder rounded,
    // about 16 significant bits in all; the running sum adds the fp32 values, which
    // differ from the two terms by about 2^-16 relative.
    auto pv_bf16_split = [&]() {
      u32x4 pb[RB], pb_lo[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        uint32_t pw[4], pw_lo[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t x = __float_as_uint(pr[b][2 * u]), y = __float_as_uint(pr[b][2 * u + 1]);
          pw[u] = (x >> 16) | (y & 0xffff0000u);
          pw_lo[u] = to_store2<kBF16>(pr[b][2 * u] - __uint_as_float(x & 0xffff0000u),
                                      pr[b][2 * u + 1] - __uint_as_float(y & 0xffff0000u));
        }
        l[b] = l[b] * alpha[b] + (((pr[b][0] + pr[b][1]) + (pr[b][2] + pr[b][3])) +
                                  ((pr[b][4] + pr[b][5]) + (pr[b][6] + pr[b][7])));
        pb[b] = u32x4{pw[0], pw[1], pw[2], pw[3]};
        pb_lo[b] = u32x4{pw_lo[0], pw_lo[1], pw_lo[2], pw_lo[3]};
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4 a = vfrag(j);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, pb[b]), acc[b][j], 0, 0, 0);
          acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, pb_lo[b]), acc[b][j], 0, 0, 0);
        }
      }
    };
    if constexpr (DT == kF32) pv_f32();
    else if constexpr (DT == kF16 || (PVH && !SAFE)) pv_f16();
    else pv_bf16_split();
  };

  // pool byte offsets of this lane's tokens from their table entries
  auto offsets = [&](const int (&tb)[NT], const int (&to)[NT], size_t (&off)[NT]) {
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      int bk = tb[k];
      bk = bk < 0 ? 0 : (bk >= p.num_blocks ? p.num_blocks - 1 : bk);
      off[k] = ((size_t)bk * B + to[k]) * slot_bytes + kv_off;
    }
  };
  auto load_rows = [&](u32x4 (&x)[KL], const void* cache, const size_t (&off)[NT]) {
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        x[k * CPT + c] = *reinterpret_cast<const u32x4*>((const char*)cache + off[k] + my_chunk(c) * 16);
  };

  if constexpr (SPLIT) {
    // every fourth tile, one set of registers.  Per tile: stage its V in the wave's
    // LDS region, start the wave's next V, multiply with this tile's K (registers),
    // start the next K and the table entries of the tile after that
    const int kstep = 4;
    int tb[NT], to[NT];
    size_t off[NT];
    if (wave < ntiles) {
      fetch_table(tb, to, tile_map(t_begin + wave * kTile));
      offsets(tb, to, off);
      load_rows(vr[0], p.v_cache, off);
      load_rows(kr[0], p.k_cache, off);
      if (wave + kstep < ntiles) fetch_table(tb, to, tile_map(t_begin + (wave + kstep) * kTile));
    }
    for (int k = wave; k < ntiles; k += kstep) {
      const int t0 = t_begin + k * kTile;
      const bool more = k + kstep < ntiles;
      store_kv(std::false_type{}, kr[0], vr[0], nullptr, ldsV);
      if (more) {
        offsets(tb, to, off);
        load_rows(vr[0], p.v_cache, off);
      }
      qk([&](int h, int c) { return kr[0][h * NKC + c]; });
      if (more) load_rows(kr[0], p.k_cache, off);
      if (k + 2 * kstep < ntiles) fetch_table(tb, to, tile_map(t0 + 2 * kstep * kTile));
      __builtin_amdgcn_wave_barrier();   // V stores above are read by other lanes below
      softmax_pv(std::false_type{}, t0, tile_map(t0), ldsV);
      __builtin_amdgcn_wave_barrier();   // V reads above before the next stores
    }
  } else {
    // all tiles, two sets of registers and two LDS buffers: while tile k is computed,
    // the rows of tiles k + 1 and k + 2 and the table entries of tile k + 3 are on
    // their way.  Tile k goes to buffer k % 2, whose last readers (tile k - 2) have
    // all passed the barrier of tile k - 1, so one barrier per tile suffices.
    auto run_plain = [&](auto safe_c) {
      int tb[2][NT], to[2][NT];
      auto step = [&](int k, char* buf, u32x4 (&xk)[KL], u32x4 (&xv)[KL], const int (&tbc)[NT],
                      const int (&toc)[NT], int (&tbn)[NT], int (&ton)[NT]) {
        const int t0 = t_begin + k * kTile;
        char* const kb = buf;
        char* const vb = buf + S::KBYTES;
        store_kv(safe_c, xk, xv, kb, vb);
        __syncthreads();
        if (k + 3 < ntiles) fetch_table(tbn, ton, tile_map(t0 + 3 * kTile));
        if (k + 2 < ntiles) {
          size_t off[NT];
          offsets(tbc, toc, off);
          load_rows(xk, p.k_cache, off);
          load_rows(xv, p.v_cache, off);
        }
        qk([&](int h, int c) {
          return *reinterpret_cast<const u32x4*>(kb + (16 * h + col) * S::KSTRIDE + chunk_of<DT, D>(c, grp) * 16);
        });
        softmax_pv(safe_c, t0, tile_map(t0), vb);
      };
      if (ntiles > 0) fetch_table(tb[0], to[0], tile_map(t_begin));
      if (ntiles > 1) fetch_table(tb[1], to[1], tile_map(t_begin + kTile));
      for (int i = 0; i < 2; ++i) {
        if (i < ntiles) {
          size_t off[NT];
          offsets(tb[i], to[i], off);
          load_rows(kr[i], p.k_cache, off);
          load_rows(vr[i], p.v_cache, off);
        }
      }
      if (ntiles > 2) fetch_table(tb[0], to[0], tile_map(t_begin + 2 * kTile));
      for (int k = 0; k < ntiles; k += 2) {
        step(k, lds, kr[0], vr[0], tb[0], to[0], tb[1], to[1]);
        if (k + 1 < ntiles) step(k + 1, lds + S::LDS, kr[1], vr[1], tb[1], to[1], tb[0], to[0]);
      }
    };
    // Pipelined loop (16-bit types), three LDS buffers.  Entering step k, tile k's scores
    // are in registers (masked if it needs a mask) and `resc` says whether some row's
    // reference must move for them.  Step k fetches the table entries of tile k + 4, stages
    // tile k + 1 in buffer (k + 1) mod 3 and passes one barrier; moves the references and
    // rescales the accumulators if `resc` (rare); then two branch-free stretches: tile k + 1's
    // scores with tile k's weights, and tile k's P.V with the loads of tile k + 3, tile
    // k + 1's mask (last tiles only) and its lanes' maxima, each matrix instruction followed
    // by a share of the vector work, so that the matrix unit runs while the vector unit
    // works.  Buffer j mod 3 is written again at step j + 2, after every wave passed the
    // barrier of step j + 1 and so finished step j, its last reader.  A tile index past the
    // last stands for the last tile (loaded, staged and scored again, never used), so the
    // stretch does not branch on the count.  A zero scale makes every visible score 0 (the
    // masked variant runs on every tile, and the softmax with scale 1), so the exponent's
    // argument is never -inf * 0.
    auto run_pipelined = [&](auto safe_c) {
      constexpr bool SAFE = decltype(safe_c)::value;
      if (ntiles <= 0) return;
      const bool zero_scale = sl2 == 0.f;
      const float sl2e = zero_scale ? 1.f : sl2;
      auto tmap = [&](int k) { return tile_map(t_begin + min(k, ntiles - 1) * kTile); };
      auto buf = [&](int k) { return lds + (k % 3) * S::LDS; };
      // tiles 0 .. nwhole - 1 are full and every row sees all of their tokens
      const int wl = min(pos_lo, t_end - 1) - t_begin - (kTile - 1);
      const int nwhole = zero_scale ? 0 : (wl >= 0 ? min(ntiles, wl / kTile + 1) : 0);
      constexpr int NQK = RB * 2 * NKC;                    // matrix instructions of one tile's scores
      int tb[2][NT], to[2][NT];
      f32x4 sA[RB][2], sB[RB][2];
      // running sums as matrix products (P times a block of ones), so they come out summed
      // over the row's four lanes
      f32x4 lacc[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) lacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      bool resc = false;
      auto load_tile = [&](const int (&tbx)[NT], const int (&tox)[NT], u32x4 (&xk)[KL], u32x4 (&xv)[KL]) {
        size_t off[NT];
        offsets(tbx, tox, off);
        load_rows(xk, p.k_cache, off);
        load_rows(xv, p.v_cache, off);
      };
      auto scores = [&](f32x4 (&dst)[RB][2], const char* kb) {
        qk_to(dst, [&](int h, int c) {
          return *reinterpret_cast<const u32x4*>(kb + (16 * h + col) * S::KSTRIDE + chunk_of<DT, D>(c, grp) * 16);
        });
      };
      // tile k's mask on raw scores: row b sees tile token u iff u < count and t0 + u <= pos[b]
      // (a tile past the last sees nothing)
      auto mask = [&](f32x4 (&sc)[RB][2], int k) {
        const int t0 = t_begin + k * kTile;
        const int cnt = min(kTile, t_end - t0);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const int lim = min(pos[b] - t0, cnt - 1);
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sc[b][h][i] = 16 * h + 4 * grp + i <= lim ? (zero_scale ? 0.f : sc[b][h][i]) : -__builtin_inff();
        }
      };
      // A row's reference moves only when a tile's scores exceed it by more than kLazyMax,
      // and then for every row of the wave at once (as in softmax_pv).  The test needs only
      // each lane's own maximum lmx: any lane over the bound sets resc for the wave.  The
      // moves (the maxima over each row's four lanes, new references, rescaled accumulators)
      // happen in the rare branch at the start of the next step, before the tile's weights.
      float lmx[RB];
      auto test_grow = [&]() {
        bool grow = false;
#pragma unroll
        for (int b = 0; b < RB; ++b) grow = grow || lmx[b] * sl2e > m[b] + kLazyMax;
        resc = __any(grow);
      };
      auto move_refs = [&]() {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const float mn = vmax(m[b], max_over_groups_nan(lmx[b]) * sl2e);
          const float alpha = fast_exp2(m[b] - mn);
          m[b] = mn;
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[b][j] *= alpha;
          lacc[b] *= alpha;
        }
      };
      auto maxima = [&](f32x4 (&sc)[RB][2]) {
#pragma unroll
        for (int b = 0; b < RB; ++b) lmx[b] = vmax8(sc[b][0], sc[b][1]);
        test_grow();
      };
      auto mfma16 = [&](const u32x4& x, const u32x4& y, const f32x4& c) {
        if constexpr (DT == kBF16)
          return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
        else
          return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
      };
      u32x4 pb[RB], pb_lo[RB];
      const uint32_t vlane = (4 * grp + (col >> 2)) * S::VSTRIDE + (4 * (col & 3)) * 2;
      const uint32_t slot32 = (uint32_t)slot_bytes, blk32 = (uint32_t)(slot_bytes * B);
      const uint32_t lane_kv = (uint32_t)kv_off + (uint32_t)my_chunk(0) * 16;
      const u32x4 ones16 = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};    // fp16 1.0
      const u32x4 onesb16 = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0
      // One step.  The two products are written as chunks of one matrix instruction (two for
      // the two-term P.V) and a share of the vector work, fenced so that the compiler keeps
      // the order; the matrix unit runs each instruction while the vector unit works.
      auto step = [&](auto mask_next_c, int k, f32x4 (&scur)[RB][2], f32x4 (&snext)[RB][2], u32x4 (&xk)[KL],
                      u32x4 (&xv)[KL], const int (&tbl)[NT], const int (&tol)[NT], int (&tbf)[NT], int (&tof)[NT]) {
        constexpr bool MASK_NEXT = decltype(mask_next_c)::value;
        char* const bn = buf(k + 1);
        fetch_table(tbf, tof, tmap(k + 4));
        store_kv(safe_c, xk, xv, bn, bn + S::KBYTES);   // tile k + 1
        __syncthreads();
        if (resc) move_refs();
        __builtin_amdgcn_sched_barrier(0);

        // Part 1: tile k + 1's scores, chunk i = (c, h, b), with tile k's weights.  The weights
        // of a pair of scores take two half-steps: two exponentials, then the packing.
        // K fragments of step c are read one step ahead
        u32x4 kf[2][NKC];
        auto kread = [&](int c) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            kf[h][c] = *reinterpret_cast<const u32x4*>(bn + (16 * h + col) * S::KSTRIDE + chunk_of<DT, D>(c, grp) * 16);
        };
#pragma unroll
        for (int b = 0; b < RB; ++b) snext[b][0] = snext[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        float pr[RB][8];
        uint32_t pw[RB][4], pw_lo[RB][4];
        auto weight_half = [&](int hs) {
          const int pair = hs >> 1, b = pair >> 2, u = pair & 3;
          const int h = u >> 1, i0 = 2 * (u & 1);
          if ((hs & 1) == 0) {
            pr[b][2 * u] = fast_exp2(fmaf(scur[b][h][i0], sl2e, -m[b]));
            pr[b][2 * u + 1] = fast_exp2(fmaf(scur[b][h][i0 + 1], sl2e, -m[b]));
          } else if constexpr (!SAFE) {
            pw[b][u] = to_store2<kF16>(pr[b][2 * u], pr[b][2 * u + 1]);
          } else {
            const uint32_t x = __float_as_uint(pr[b][2 * u]), y = __float_as_uint(pr[b][2 * u + 1]);
            pw[b][u] = (x >> 16) | (y & 0xffff0000u);
            pw_lo[b][u] = to_store2<kBF16>(pr[b][2 * u] - __uint_as_float(x & 0xffff0000u),
                                           pr[b][2 * u + 1] - __uint_as_float(y & 0xffff0000u));
          }
        };
        constexpr int HS = RB * 8;                     // half-steps of the weights
        constexpr int PER1 = (HS + NQK - 1) / NQK;
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
          const int c = i / (2 * RB), h = (i / RB) % 2, b = i % RB;
          if (i == 0) kread(0);
          if (i % (2 * RB) == 0 && c + 1 < NKC) kread(c + 1);
          snext[b][h] = mfma16(kf[h][c], qf[b][c], snext[b][h]);
#pragma unroll
          for (int q = 0; q < PER1; ++q)
            if (i * PER1 + q < HS) weight_half(i * PER1 + q);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          pb[b] = u32x4{pw[b][0], pw[b][1], pw[b][2], pw[b][3]};
          if constexpr (SAFE) pb_lo[b] = u32x4{pw_lo[b][0], pw_lo[b][1], pw_lo[b][2], pw_lo[b][3]};
        }

        // Part 2: tile k's P.V, chunk j = one head_dim block (every row block), with tile k + 1's
        // mask (last tiles only), row maxima and settled references, and the loads of tile k + 3
        // into the registers just staged.  V fragments are read two chunks ahead.
        // one address register per step, so that the fragments' offsets stay immediates
        uint32_t voff = (uint32_t)((k % 3) * S::LDS + S::KBYTES) + vlane;
        asm volatile("" : "+v"(voff));
        const char* vbase = lds + voff;
        u32x4 vf[NJ];
        auto vread = [&](int j) {
          const s16x4 a0 = lds_read_tr16(vbase + 32 * j);
          const s16x4 a1 = lds_read_tr16(vbase + 16 * S::VSTRIDE + 32 * j);
          vf[j] = __builtin_bit_cast(u32x4, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        const int t1 = t_begin + (k + 1) * kTile;
        constexpr int NMASK = MASK_NEXT ? RB : 0;
        constexpr int NW = NMASK + RB + 1 + NT;       // pieces of vector work
        auto work = [&](int w0) {
          // the loads first, so that they have most of a step more to arrive
          const int w = w0 < NT ? NMASK + RB + 1 + w0 : w0 - NT;
          if (w < NMASK) {                              // mask of row block w
            const int b = w;
            const int lim = min(pos[b] - t1, min(kTile, t_end - t1) - 1);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                snext[b][h][i] = 16 * h + 4 * grp + i <= lim ? (zero_scale ? 0.f : snext[b][h][i]) : -__builtin_inff();
          } else if (w < NMASK + RB) {                  // a row block's maximum over its lane
            const int b = w - NMASK;
            lmx[b] = vmax8(snext[b][0], snext[b][1]);
          } else if (w == NMASK + RB) {                 // does any reference have to move?
            test_grow();
          } else {                                      // the lane's token of tile k + 3: K and V rows
            const int t = w - NMASK - RB - 1;
            const int bk = min(max(tbl[t], 0), p.num_blocks - 1);
            // block * block bytes (one 32x32 -> 64-bit multiply-add) + slot row and chunk offset
            // (block bytes < 2^32 and slot bytes < 2^24, checked by the host)
            const uint32_t lo = __umul24((uint32_t)tol[t], slot32) + lane_kv;
            const size_t off = (size_t)(uint32_t)bk * blk32 + lo;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
              xk[t * CPT + c] = *reinterpret_cast<const u32x4*>((const char*)p.k_cache + off + 128 * c);
              xv[t * CPT + c] = *reinterpret_cast<const u32x4*>((const char*)p.v_cache + off + 128 * c);
            }
          }
        };
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (j == 0) {
#pragma unroll
            for (int r = 0; r < 2 && r < NJ; ++r) vread(r);
          }
          if (j + 2 < NJ) vread(j + 2);
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            if constexpr (!SAFE) {   // fp16 V (stored or widened) and fp16 weights
              acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, vf[j]),
                                                                 __builtin_bit_cast(f16x8, pb[b]), acc[b][j], 0, 0, 0);
            } else {
              acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[j]),
                                                                  __builtin_bit_cast(bf16x8, pb[b]), acc[b][j], 0, 0, 0);
              acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[j]),
                                                                  __builtin_bit_cast(bf16x8, pb_lo[b]), acc[b][j], 0, 0, 0);
            }
          }
          if (j == NJ - 1) {                            // the running sums
#pragma unroll
            for (int b = 0; b < RB; ++b) {
              if constexpr (!SAFE) {
                lacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ones16),
                                                                 __builtin_bit_cast(f16x8, pb[b]), lacc[b], 0, 0, 0);
              } else {
                lacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, onesb16),
                                                                  __builtin_bit_cast(bf16x8, pb[b]), lacc[b], 0, 0, 0);
                lacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, onesb16),
                                                                  __builtin_bit_cast(bf16x8, pb_lo[b]), lacc[b], 0, 0, 0);
              }
            }
          }
#pragma unroll
          for (int w = j * NW / NJ; w < (j + 1) * NW / NJ; ++w) work(w);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      fetch_table(tb[0], to[0], tmap(0));
      fetch_table(tb[1], to[1], tmap(1));
      load_tile(tb[0], to[0], kr[0], vr[0]);
      load_tile(tb[1], to[1], kr[1], vr[1]);
      fetch_table(tb[0], to[0], tmap(2));
      store_kv(safe_c, kr[0], vr[0], lds, lds + S::KBYTES);   // tile 0 -> buffer 0
      __syncthreads();
      // tile 3's table entries before tile 2's rows: the order of a step (table entries of
      // tile k + 4 before the rows of tile k + 3), so that the waits the compiler places at the
      // loop head, which must hold for the first entry too, wait only for what a step needs
      fetch_table(tb[1], to[1], tmap(3));
      load_tile(tb[0], to[0], kr[0], vr[0]);                    // tile 2
      scores(sA, lds);
      if (nwhole == 0) mask(sA, 0);
      maxima(sA);
      // whole tiles with a whole successor, in pairs; then the rest with masks
      const int nfast = max(0, nwhole - 1) & ~1;
      int k = 0;
      for (; k < nfast; k += 2) {
        step(std::false_type{}, k, sA, sB, kr[1], vr[1], tb[1], to[1], tb[0], to[0]);
        step(std::false_type{}, k + 1, sB, sA, kr[0], vr[0], tb[0], to[0], tb[1], to[1]);
      }
      for (; k < ntiles; k += 2) {
        step(std::true_type{}, k, sA, sB, kr[1], vr[1], tb[1], to[1], tb[0], to[0]);
        if (k + 1 < ntiles) step(std::true_type{}, k + 1, sB, sA, kr[0], vr[0], tb[0], to[0], tb[1], to[1]);
      }
      // every element of a running-sum block holds the row's whole sum
#pragma unroll
      for (int b = 0; b < RB; ++b) l[b] = lacc[b][0];
    };
    auto run_tiles = [&](auto safe_c) {
      if constexpr (!PIPE) {
        run_plain(safe_c);
      } else {
        run_pipelined(safe_c);
      }
    };
    run_tiles(std::false_type{});
    if constexpr (PVH) {
      // A V value of 2^16 or more became inf in fp16, so every accumulator it reached
      // is inf or NaN (p inf, or 0 inf for a masked token).  Any non-finite accumulator
      // in the workgroup sends all four waves through the tiles again with V staged as
      // bf16 and P split into two bf16 terms (exact for every finite input; input that
      // is itself non-finite gives the same non-finite result either way).  The flag
      // words are written by every wave before the barrier and read after it.
      bool bad = false;
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) bad = bad || !__builtin_isfinite(acc[b][j][i]);
      const bool wave_bad = __any(bad);
      if (lane == 0) redo_flag[wave] = wave_bad ? 1u : 0u;
      __syncthreads();
      const uint32_t any_bad = redo_flag[0] | redo_flag[1] | redo_flag[2] | redo_flag[3];
      if (__builtin_amdgcn_readfirstlane(any_bad) != 0u) {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          m[b] = kNegBig;
          l[b] = 0.f;
        }
        run_tiles(std::true_type{});
      }
    }
  }

  // each row's sum over its four lanes; lane (grp, col) holds head_dim 16 j + 4 grp + i
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if constexpr (!PIPE) {   // (the pipelined loop's sums are whole already)
      l[b] += __shfl_xor(l[b], 16);
      l[b] += __shfl_xor(l[b], 32);
    }
  }
  if constexpr (SPLIT) {
    // merge the four waves' results for the same 16 rows: wave w's (m, l) and
    // accumulator go to LDS region w; then wave w combines head_dim blocks j = w (mod 4)
    __syncthreads();   // every wave is done with its V region
    float* mine = reinterpret_cast<float*>(lds) + wave * 16 * (D + 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j) *reinterpret_cast<f32x4*>(mine + col * D + 16 * j + 4 * grp) = acc[0][j];
    if (grp == 0) {
      mine[16 * D + 2 * col] = m[0];
      mine[16 * D + 2 * col + 1] = l[0];
    }
    __syncthreads();
    if (!row_ok[0]) return;
    const float* part = reinterpret_cast<const float*>(lds);
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, part[w * 16 * (D + 2) + 16 * D + 2 * col]);
    float wt[4], Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* src = part + w * 16 * (D + 2) + 16 * D + 2 * col;
      wt[w] = fast_exp2(src[0] - M);
      Lsum += wt[w] * src[1];
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    for (int j = wave; j < NJ; j += 4) {
      f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w)
        o += wt[w] * *reinterpret_cast<const f32x4*>(part + w * 16 * (D + 2) + col * D + 16 * j + 4 * grp);
      if (p.parts == 1) {
        store4<DT>((char*)p.out + out_row[0] * S::ROWB + (16 * j + 4 * grp) * EB, o * inv);
      } else if (ntiles > 0) {  // the merge reads no accumulator of an empty partition
        const size_t slot = out_row[0] * p.parts + it.part;
        *reinterpret_cast<f32x4*>(p.ws_acc + slot * D + 16 * j + 4 * grp) = o;
      }
    }
    if (p.parts > 1 && wave == 0 && grp == 0) {
      const size_t slot = out_row[0] * p.parts + it.part;
      *reinterpret_cast<u32x2*>(p.ws_ml + slot * 2) = u32x2{__float_as_uint(M), __float_as_uint(Lsum)};
    }
  } else {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (!row_ok[b]) continue;
      if (p.parts == 1) {
        const float inv = l[b] > 0.f ? 1.f / l[b] : 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          store4<DT>((char*)p.out + out_row[b] * S::ROWB + (16 * j + 4 * grp) * EB, acc[b][j] * inv);
      } else {
        const size_t slot = out_row[b] * p.parts + it.part;
        if (ntiles > 0) {  // the merge reads no accumulator of an empty partition
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            *reinterpret_cast<f32x4*>(p.ws_acc + slot * D + 16 * j + 4 * grp) = acc[b][j];
        }
        if (grp == 0)
          *reinterpret_cast<u32x2*>(p.ws_ml + slot * 2) = u32x2{__float_as_uint(m[b]), __float_as_uint(l[b])};
      }
    }
  }
}

// Merge the partitions of every (query row, head), in partition order:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
// One wave per (row, head); lane i handles head_dim elements i, i + 64.
template <int DT, int D>
__global__ __launch_bounds__(256) void multi_query_merge_kernel(MultiQueryParams p) {
  const long long rh = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= (long long)p.total_q * p.num_heads) return;
  const int lane = threadIdx.x & 63;
  const float* ml = p.ws_ml + (size_t)rh * p.parts * 2;
  float M = kNegBig;
  for (int q = 0; q < p.parts; ++q) M = fmaxf(M, ml[2 * q]);
  constexpr int PER = D / 64;
  float o[PER] = {};
  float lsum = 0.f;
  for (int q = 0; q < p.parts; ++q) {
    if (!(ml[2 * q + 1] > 0.f)) continue;   // empty partition: no accumulator was written
    const float w = fast_exp2(ml[2 * q] - M);
    lsum += w * ml[2 * q + 1];
    const float* a = p.ws_acc + ((size_t)rh * p.parts + q) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += w * a[lane + 64 * e];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  constexpr int EB = DT == kF32 ? 4 : 2;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    char* dst = (char*)p.out + (size_t)rh * D * EB + (size_t)(lane + 64 * e) * EB;
    if constexpr (DT == kF32) *reinterpret_cast<float*>(dst) = o[e] * inv;
    else *reinterpret_cast<uint16_t*>(dst) = to_store<DT>(o[e] * inv);
  }
}

template <int DT, int D>
void pick_d(int rows, bool shared, const void** main, const void** merge) {
  *merge = reinterpret_cast<const void*>(&multi_query_merge_kernel<DT, D>);
  if constexpr (DT != kF32) {
    if (shared) {
      *main = reinterpret_cast<const void*>(&multi_query_kernel<DT, D, true, true, 1>);
      return;
    }
    if (rows == 16) {
      *main = reinterpret_cast<const void*>(&multi_query_kernel<DT, D, true, false, 1>);
      return;
    }
  }
  if (rows == 128) *main = reinterpret_cast<const void*>(&multi_query_kernel<DT, D, false, false, 2>);
  else *main = reinterpret_cast<const void*>(&multi_query_kernel<DT, D, false, false, 1>);
}

template <int DT>
bool pick_dt(int head_dim, int rows, bool shared, const void** main, const void** merge) {
  if ((rows == 16 || shared) && DT == kF32) return false;
  if (head_dim == 64) {
    pick_d<DT, 64>(rows, shared, main, merge);
    return true;
  }
  if (head_dim == 128) {
    pick_d<DT, 128>(rows, shared, main, merge);
    return true;
  }
  return false;
}

}  // namespace

const void* multi_query_order_kernel(bool shared) {
  return shared ? reinterpret_cast<const void*>(&item_order_kernel<true>)
                : reinterpret_cast<const void*>(&item_order_kernel<false>);
}

bool multi_query_kernels(int dtype, int head_dim, int rows, bool shared, const void** main,
                         const void** merge) {
  if (rows != 16 && rows != 64 && rows != 128) return false;
  switch (dtype) {
    case kF32: return pick_dt<kF32>(head_dim, rows, shared, main, merge);
    case kF16: return pick_dt<kF16>(head_dim, rows, shared, main, merge);
    case kBF16: return pick_dt<kBF16>(head_dim, rows, shared, main, merge);
    default: return false;
  }
}

}  // namespace pagedkv
