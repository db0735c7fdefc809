// Paged decode attention kernels for gfx950 (CDNA4), one template instantiated per
// element type in decode_{f32,f16,bf16}.hip.
//
// What is computed: for each sequence and query head, softmax(scale * q.K^T) V
// over the sequence's tokens, whose K/V rows sit in fixed-size physical blocks
// reached through the sequence's block table; the softmax is normalised across
// blocks by a running maximum and running sum merged block by block
// ("LLM 注意力与计算内核精读笔记 · 05 PagedAttention 与 KV 显存管理", §4; the
// dense formula with 1/sqrt(d) is in "vLLM 是什么 PagedAttention 解决了什么",
// section "2）PagedAttention 算子").
//
// Work decomposition (split.h)
//   The step's work is cut into 16-token tiles of (sequence, KV head) pairs and
//   every launched wave takes the same number of consecutive tiles, so each reads
//   the same number of K/V bytes whatever the length mix.  There is one wave per
//   SIMD: four independent 64-lane waves per workgroup, one workgroup per CU.  A pair that falls entirely
//   inside one wave is finished there; a pair cut by a wave boundary leaves one
//   partial result per piece, and reduce_kernel merges them.  Every query head of
//   a KV head's group (g = num_heads / num_kv_heads <= GP) is handled by the same
//   wave, so each K/V row is read from HBM once.
//
// Prologue
//   Each wave loads the lengths of all sequences (512 at a time, in one round
//   trip) and sums their tile counts to get the total T, keeping each sequence's
//   length and tile prefix sum in LDS, where it locates the pair and tile its range
//   begins with.  Sequences of length 0 have no tiles; their zero outputs are
//   written by wave s mod (number of waves) during that pass.
//
// Lane roles inside a segment (lane = 16 * grp + col, grp = 0..3, col = 0..15)
//   q.K^T on the matrix cores: v_mfma_f32_16x16x32_{bf16,f16} (or 16x16x4_f32)
//     with A = the tile's K rows (row = token col, this lane's 16-byte chunks
//     4c + grp of the row) and B = the group's query rows padded to 16 columns
//     (column = head col, same chunks).  Any fixed assignment of head_dim
//     positions to MFMA k-slots gives the same dot products, so the chunking
//     only has to match between A and B.  The result lands as
//     S[token 4*grp + r][head col], r = 0..3, in lane (grp, col).
//   P.V on the matrix cores (16-bit types, groups of 3 or more query heads):
//     O^T += V^T P^T with v_mfma_f32_16x16x16_{bf16,f16}, one product per
//     element e of the lane's V slice: the A operand is element col * head_dim/16
//     + e of the lane's four token rows (gathered with v_perm), the B operand is
//     the lane's own four weights, so no weight moves between lanes.  Lane
//     (grp, col) ends with head col over elements (4*grp + r) * head_dim/16 + e.
//     All 16 tokens of a tile meet in one sum, so every head keeps one reference
//     maximum for the four row groups (row swaps v_permlane{32,16}_swap), moved
//     only when a tile exceeds it by 2^8: weights stay below 256 and the
//     accumulators are rescaled on few tiles.  bf16 weights are split into two
//     bf16 terms (about 16 significant bits), fp16 weights are rounded once.
//   P.V on the vector ALU (fp32, and groups of 1 or 2): lane (grp, col) keeps its
//     own running max m and sum l for head col over the tokens 4*grp + r of
//     every tile, i.e. four independent streams per head, merged once at the end
//     of the segment.  It owns head_dim/16 consecutive elements (at col *
//     head_dim/16) of tokens 4*grp + j, j = 0..3, and accumulates acc[h][.] for
//     every head h of the group.  The weight p of (head h, token 4*grp + j) sits
//     in lane (grp, h); DPP row_newbcast:h broadcasts it to the 16 lanes of the
//     row -- no LDS, no barrier.
//   Block ids: lane i holds the id of the segment's block 64 w + i for the
//     current window w (v_readlane picks it per tile) and the next 64 ids are
//     fetched a window ahead, so the two-tile pipeline runs through a whole
//     segment without draining at window boundaries.
//
// Append variant (APPEND, for pa_decode_append): the newest token of every pair
// (position L - 1) is read from the new rows passed with the call instead of its
// slot, and the merge kernel's extra workgroups store those rows into the slot
// after this kernel has finished.  The plain variant's code is unchanged by it.
//
// Logits are taken in base 2 (scale * log2 e folded in), so every exponential is
// one v_exp_f32.  Running maxima start at a finite -1e30 so that a stream with
// no valid token yet never forms inf - inf.  Tokens past the end of a window in
// its last tile are redirected to the window's last token before loading (so no
// unused slot is ever read) and their scores are replaced by -inf with a select,
// which makes their weights exactly 0.
#pragma once

#include <type_traits>

#include "decode_params.h"
#include "split.h"

namespace pagedkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;
#ifndef PA_DECODE_PIPE
#define PA_DECODE_PIPE 2
#endif
// K/V tiles in flight per wave (3 measured no faster than 2 on the Llama-3-8B shape)
constexpr int kDecodePipe = PA_DECODE_PIPE;
#ifndef PA_DECODE_MPV_MIN_GP
#define PA_DECODE_MPV_MIN_GP 4
#endif
// P.V on the matrix cores for 16-bit types from this padded group size on; smaller
// groups keep it on the vector ALU (with one or two heads most of the 16 product
// rows would be padding).
template <int DT, int GP>
constexpr bool kMatrixPV = DT != kF32 && GP >= PA_DECODE_MPV_MIN_GP;
// A reference maximum moves only when a tile's maximum exceeds it by more than this
// (log2 units), so weights stay below 2^8 and the accumulators are rescaled rarely.
constexpr float kLazyMax = 8.0f;

template <int DT>
struct Elem {
  static constexpr int bytes = DT == kF32 ? 4 : 2;
};

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// Value of lane SRC of this lane's 16-lane row (DPP row_newbcast).
template <int SRC>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, 0x150 + SRC, 0xF, 0xF, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum over lanes i, i ^ 16, i ^ 32 and i ^ 48 (the four 16-lane rows) with the
// gfx950 row swaps: swapping a value with a copy of itself leaves one lane of each
// pair in each result, so the larger of the two is the pair's maximum.
__device__ __forceinline__ float max_over_rows(float x) {
  // (left-leaning chains, so that each step is one v_max3 and the swapped values are not
  // first passed through a canonicalising maximum of their own)
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(fmaxf(x, __uint_as_float(a[0])), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(fmaxf(x, __uint_as_float(b[0])), __uint_as_float(b[1]));
}

// Two floats rounded to nearest even in a 16-bit type, the first in the low half.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  if constexpr (DT == kBF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
  }
}

// One 16x16x16 product on the matrix cores, 16-bit inputs, fp32 accumulate.
template <int DT>
__device__ __forceinline__ f32x4 mfma16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, u32x2{a0, a1}),
                                                     __builtin_bit_cast(s16x4, u32x2{b0, b1}), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, u32x2{a0, a1}),
                                                 __builtin_bit_cast(f16x4, u32x2{b0, b1}), c, 0, 0, 0);
}

// Inclusive prefix sum over the 64 lanes, in registers: shifts by 1, 2, 4, 8
// inside each 16-lane row (lanes shifted in from outside the row read 0), then
// lane 15 of each row is added to the next row and lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false); // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false); // row_bcast:31 -> rows 2, 3
  return x;
}

// Sum over the 64 lanes, the same in every lane.
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan(x), 63);
}

// Length of sequence s as the kernels use it: clamped to [0, max_seq_len].
__device__ __forceinline__ int seq_len_at(const DecodeParams& p, int s) {
  const int L = p.seq_lens[s];
  return L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
}

// Widen NW packed dwords of element type DT to floats (element 2i is the low half).
template <int DT, int NW>
__device__ __forceinline__ void unpack(const uint32_t (&w)[NW], float (&f)[NW * 4 / Elem<DT>::bytes]) {
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if constexpr (DT == kF32) {
      f[i] = __uint_as_float(w[i]);
    } else if constexpr (DT == kBF16) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    } else {
      f16x2 h = __builtin_bit_cast(f16x2, w[i]);
      f[2 * i] = (float)h.x;
      f[2 * i + 1] = (float)h.y;
    }
  }
}

// Round-to-nearest-even store of N floats as element type DT.
template <int DT, int N>
__device__ __forceinline__ void store_row(void* dst, const float (&v)[N]) {
  if constexpr (DT == kF32) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 4) {
        u32x4 w = {__float_as_uint(v[i]), __float_as_uint(v[i + 1]), __float_as_uint(v[i + 2]),
                   __float_as_uint(v[i + 3])};
        reinterpret_cast<u32x4*>(dst)[i / 4] = w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) reinterpret_cast<float*>(dst)[i] = v[i];
    }
  } else {
    uint32_t w[(N + 1) / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      uint16_t lo, hi;
      if constexpr (DT == kBF16) {
        lo = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i]);
        hi = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i + 1]);
      } else {
        lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
        hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
      }
      w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N / 8; ++i)
        reinterpret_cast<u32x4*>(dst)[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
    } else if constexpr (N == 4) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
    } else if constexpr (N == 2) {
      *reinterpret_cast<uint32_t*>(dst) = w[0];
    } else {
      static_assert(N == 1, "row piece of 1, 2, 4 or a multiple of 8 elements");
      if constexpr (DT == kBF16) *reinterpret_cast<__bf16*>(dst) = (__bf16)v[0];
      else *reinterpret_cast<_Float16*>(dst) = (_Float16)v[0];
    }
  }
}

// K/V loads.  STREAM: the non-temporal hint (the `nt` bit), so the streamed lines are
// not kept in the caches; the right policy when every row is read once per call (the
// Llama-3-8B decode: 394 against 430 µs per call).  Otherwise the default policy, which
// lets rows that several sequences of the batch share hit in L2 and the Infinity Cache.
template <bool STREAM>
__device__ __forceinline__ u32x4 load16_kv(const char* src) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
  else return *reinterpret_cast<const u32x4*>(src);
}

template <bool STREAM, int NW>
__device__ __forceinline__ void load_dwords(const char* src, uint32_t (&w)[NW]) {
  static_assert(NW == 2 || NW % 4 == 0, "row slice must be 8 or a multiple of 16 bytes");
  if constexpr (NW == 2) {
    u32x2 x;
    if constexpr (STREAM) x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
    else x = *reinterpret_cast<const u32x2*>(src);
    w[0] = x.x;
    w[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      u32x4 x = load16_kv<STREAM>(src + 16 * i);
      w[4 * i] = x.x;
      w[4 * i + 1] = x.y;
      w[4 * i + 2] = x.z;
      w[4 * i + 3] = x.w;
    }
  }
}

template <int DT, int D, int BS, int GP, bool APPEND, bool STREAM, bool ROWS>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int ROWB = D * EB;       // bytes of one (token, KV head) row
  constexpr int NKC = ROWB / 64;     // 16-byte K chunks per lane per tile
  constexpr int VE = D / 16;         // V elements per lane per token
  constexpr int VW = VE * EB / 4;    // V dwords per lane per token
  static_assert(ROWB % 64 == 0 && (BS == 8 || BS == 16 || BS == 32), "shape");
  static_assert(!ROWS || (kMatrixPV<DT, GP> && !APPEND), "multi-query rows use the matrix-core P.V");

  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);  // waves never talk to each other
  const int launched = p.num_waves;
  if (w >= launched) return;
  const int N = p.num_seqs;
  const int Hkv = p.num_kv_heads;
  const int g = p.group;

  // Tiles of sequence s as seen by this lane (0 past the batch).
  auto lane_tiles = [&](int s) { return s < N ? tiles_of(seq_len_at(p, s)) : 0; };

  // This wave's LDS copy of the lengths and of the tiles before each sequence (one
  // KV head's worth: pair (s, kv) starts at tile Hkv * pre[s] + kv * n_s).
  __shared__ int lds_pre[4][kLdsSeqs + 1];
  __shared__ int lds_len[4][kLdsSeqs];
  int* const pre = lds_pre[threadIdx.x >> 6];
  int* const lenl = lds_len[threadIdx.x >> 6];
  bool in_lds = N <= kLdsSeqs;
  // ROWS: the query starts q_start[0..N] as well, loaded with the lengths
  __shared__ int lds_qs[4][ROWS ? kLdsSeqs + 1 : 1];
  int* const qsl = lds_qs[threadIdx.x >> 6];
  int q_end = 0;
  if constexpr (ROWS) q_end = p.q_start[N];

  // Total tiles of the step (and, for a batch that fits, every sequence's length and
  // exclusive tile prefix sum in LDS).  The lengths of kLenRound * 64 sequences are
  // loaded at once, unconditionally (indices past the batch read its last length and
  // are masked afterwards), so the pass costs one memory round trip per round rather
  // than one per 64 sequences.
  long long seq_tiles = 0;
  {
    constexpr int kLenRound = 8;
    for (int c0 = 0; c0 < N; c0 += 64 * kLenRound) {
      int raw[kLenRound], rawq[kLenRound];
#pragma unroll
      for (int i = 0; i < kLenRound; ++i) {
        raw[i] = p.seq_lens[min(c0 + 64 * i + lane, N - 1)];
        if constexpr (ROWS) rawq[i] = p.q_start[min(c0 + 64 * i + lane, N - 1)];
      }
#pragma unroll
      for (int i = 0; i < kLenRound; ++i) {
        const int c = c0 + 64 * i;
        if (c >= N) break;
        const int L = c + lane < N ? (raw[i] < 0 ? 0 : min(raw[i], p.max_seq_len)) : 0;
        const int n_cur = tiles_of(L);
        const int incl = wave_inclusive_scan(n_cur);
        if (in_lds && c + lane < N) {
          pre[c + lane] = (int)(seq_tiles + incl - n_cur);
          lenl[c + lane] = L;
          if constexpr (ROWS) qsl[c + lane] = rawq[i];
        }
        seq_tiles += __builtin_amdgcn_readlane(incl, 63);
        // outputs of empty sequences are zeros: sequence s is zeroed by wave s mod launched
        // (ROWS: an empty sequence has no query rows)
        unsigned long long empty =
            __ballot(!ROWS && c + lane < N && L == 0 && (c + lane) % launched == w);
        while (empty) {
          const int s = c + __ffsll(empty) - 1;
          empty &= empty - 1;
          u32x4* o = reinterpret_cast<u32x4*>((char*)p.out + (size_t)s * p.num_heads * ROWB);
          const int n16 = p.num_heads * ROWB / 16;
          for (int i2 = lane; i2 < n16; i2 += 64) o[i2] = u32x4{0, 0, 0, 0};
        }
      }
    }
    // prefix sums must fit in an int; the writes above complete before any read
    in_lds = in_lds && seq_tiles < (1ll << 31) - 1;
    if (in_lds && lane == 0) pre[N] = (int)seq_tiles;
    if (ROWS && in_lds && lane == 0) qsl[N] = q_end;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  }
  const long long T = seq_tiles * Hkv;
  const long long nw = waves_used(T, launched);
  const ChunkPlan plan{T, nw, effective_tail_div(T, nw, p.tail_div), p.tail_pieces};

  // Workspace header: [0] = chunks of this call (for the merge kernel), [32] =
  // counter of tail parts handed out (the merge kernel sets it back to 0).
  int* const hdr = p.ws_meta;
  int* const chunk_meta = p.ws_meta + 64;
  if (w == 0 && lane == 0) hdr[0] = (int)plan.chunks();

  // Next tail part for this wave, or -1 when all are taken.  A counter that did not
  // start at 0 (a workspace never zeroed) gives tickets outside [0, pieces * nw),
  // which hand out nothing rather than a chunk outside the plan.
  auto next_tail = [&]() -> long long {
    int ticket = 0;
    if (lane == 0) ticket = atomicAdd(hdr + 32, 1);
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    return ticket >= 0 && ticket < (long long)plan.pieces * nw ? plan.ticket_chunk(ticket) : -1;
  };

  const size_t tok_stride = (size_t)Hkv * ROWB;
  const size_t blk_bytes = (size_t)BS * tok_stride;
  const float sl2 = p.scale_log2e;
  auto lenf = [&](int s) { return in_lds ? lenl[s] : seq_len_at(p, s); };
  // ROWS: first query row of sequence s (s <= N), and this lane's row of a pair: query
  // row_i, head row_h of the KV head's group (columns at and past p.rows are padding)
  // (the host runs the rows mode only for batches whose tables fit LDS, so qsl is
  // always filled; reading it alone keeps these reads off the vector memory counter)
  auto qsf = [&](int s) { return min(max(qsl[s], 0), p.total_q); };
  const int row_i = ROWS ? col / g : 0;
  const int row_h = ROWS ? col - row_i * g : col;
  auto valid_id = [&](int id) __attribute__((always_inline)) {
    return (unsigned)id < (unsigned)p.num_blocks ? id : 0;
  };
  // rows mode: shared-prefix table entries carry more than the block id
  const int id_mask = ROWS && p.shared ? (int)kSharedIdMask : -1;
  // Raw ids of blocks 64 wi + lane of sequence s, which has nblk blocks.  They
  // are range-checked only where a tile uses them, so a prefetch never stalls on
  // its data; an id outside the pool is a contract violation and becomes 0, so no
  // access leaves the pool.
  auto fetch_ids = [&](int s, int nblk, int wi) __attribute__((always_inline)) {
    const int b = 64 * wi + lane;
    return b < nblk ? p.block_tables[(size_t)s * p.max_blocks_per_seq + b] : 0;
  };
  auto blocks_of = [&](int L) { return (L + BS - 1) / BS; };
  auto next_seq = [&](int s) {  // next non-empty sequence after s (N if none)
    int t = s + 1;
    while (t < N && lenf(t) == 0) ++t;
    return t;
  };
  // Query fragments (MFMA B operand) of pair (s, kv): head kv g + col, chunks 4c + grp.
  auto load_q = [&](u32x4 (&qf)[NKC], int s, int kv) __attribute__((always_inline)) {
    if constexpr (ROWS) {
      const int q0 = qsf(s);
      const bool ok = col < p.rows && row_i < qsf(s + 1) - q0;  // q0 + row_i < total_q
      const char* qrow = (const char*)p.q + ((size_t)(q0 + row_i) * p.num_heads + kv * g + row_h) * ROWB;
#pragma unroll
      for (int c = 0; c < NKC; ++c)
        qf[c] = ok ? *reinterpret_cast<const u32x4*>(qrow + (4 * c + grp) * 16) : u32x4{0, 0, 0, 0};
    } else {
      const char* qrow = (const char*)p.q + ((size_t)s * p.num_heads + kv * g + col) * ROWB;
#pragma unroll
      for (int c = 0; c < NKC; ++c)
        qf[c] = col < g ? *reinterpret_cast<const u32x4*>(qrow + (4 * c + grp) * 16) : u32x4{0, 0, 0, 0};
    }
  };

  struct Tile {
    u32x4 k[NKC];
    uint32_t v[4][VW];
    int vis;  // rows mode over shared-prefix groups: the table entry of the tile's block
  };

  // The wave's own head chunk first, then tail parts while any are left.
  // Without tails each wave records its own (empty) tail parts instead.
  const long long head = (long long)w * (plan.pieces + 1);
  if (plan.tail_div == 0 && w < nw && lane == 0)
    for (int r = 1; r <= plan.pieces; ++r)
      *reinterpret_cast<u32x4*>(chunk_meta + 4 * (head + r)) = u32x4{0u, 0u, 0u, 0u};
  auto next_chunk = [&]() -> long long { return plan.tail_div > 0 ? next_tail() : -1; };
  int scan_c = 0;            // block of 64 sequences where the last located chunk began
  long long scan_base = 0;   // tiles before that block
  for (long long ck = w < nw ? head : next_chunk(); ck >= 0; ck = next_chunk()) {
    const long long t0 = plan.begin(ck);
    const long long t1 = plan.begin(ck + 1);
    int meta_s = 0, meta_kv = 0, meta_parts = 0, meta_first = 0;
    // Find the pair and tile of t0: the first sequence whose tiles end past t0,
    // i.e. the last s < N with Hkv * pre[s] <= t0 (such an s is never empty).
    // From LDS: one ballot over every 64th prefix sum, then one over the 64
    // sequences of the block it picks.  Otherwise a scan 64 sequences at a time
    // (the next 64 lengths load while the current ones are scanned) that resumes
    // from the block of 64 where this wave's previous chunk began when t0 lies
    // past it.
    int s0 = -1;
    long long pair_base = 0;
    if (t0 < t1 && in_lds) {
      const int i1 = 64 * lane;
      const unsigned long long b1 = __ballot(i1 < N && (long long)pre[i1] * Hkv <= t0);
      const int k1 = 63 - __clzll(b1 | 1ull);
      const int i2 = 64 * k1 + lane;
      const unsigned long long b2 = __ballot(i2 < N && (long long)pre[i2] * Hkv <= t0);
      s0 = 64 * k1 + (63 - __clzll(b2 | 1ull));
      pair_base = (long long)pre[s0] * Hkv;
    } else if (t0 < t1) {
      if (t0 < scan_base) {
        scan_c = 0;
        scan_base = 0;
      }
      long long base = scan_base;
      int n_cur = lane_tiles(scan_c + lane);
      for (int c = scan_c; c < N; c += 64) {
        const int n_nxt = lane_tiles(c + 64 + lane);
        const int incl = wave_inclusive_scan(n_cur);
        const unsigned long long hit = __ballot(c + lane < N && base + (long long)incl * Hkv > t0);
        if (hit) {
          const int ln = __ffsll(hit) - 1;
          s0 = c + ln;
          pair_base = base + (long long)__builtin_amdgcn_readlane(incl - n_cur, ln) * Hkv;
          scan_c = c;
          scan_base = base;
          break;
        }
        base += (long long)__builtin_amdgcn_readlane(incl, 63) * Hkv;
        n_cur = n_nxt;
      }
    }
    // s0 >= 0 and 0 <= off < Hkv * n0 always for a non-empty chunk (t0 < T); the
    // tests only guard against reading past the lengths or the pool
    const int L0 = s0 >= 0 ? lenf(s0) : 0;
    int n0 = tiles_of(L0);
    const long long off = t0 - pair_base;
    if (t0 >= t1 || off < 0 || off >= (long long)Hkv * n0) n0 = 0;
    if (n0 > 0) {
      const int nt = (int)(t1 - t0);
      // Two cursors walk the chunk's tiles in pair order: `lc` two tiles ahead,
      // issuing loads, and `cc` behind it, computing.  Loads never stop at the end
      // of a pair, so the pipeline stays full across segments; the softmax state
      // is flushed when `cc` finishes a segment.
      TileCursor lc{s0, (int)(off / n0), (int)(off % n0), n0, L0};
      TileCursor cc = lc;
      // ROWS: tokens this lane's query row sees in the compute cursor's pair (query i of
      // the pair's n queries sits at position L - n + i); padding rows see them all
      // Shared-prefix groups: the owner index this lane's row answers to (its member
      // row; padding rows answer to the prefix owner and so see every tile).
      auto visible = [&](int s, int L) {
        const int nq = qsf(s + 1) - qsf(s);
        if (p.shared) return row_i < nq ? row_i : kSharedAll;
        return row_i < nq ? L - nq + row_i + 1 : L;
      };
      int c_vis = 0;
      if constexpr (ROWS) c_vis = visible(cc.s, cc.L);

      // load side: ids of lc's current window (`ids_cur`) and the next one, the
      // first two windows of lc's sequence (for its next KV head) and of the next
      // non-empty sequence (prefetched a sequence ahead)
      int l_seq = s0, l_nblk = blocks_of(L0);
      int lw = (kTileTokens * lc.j / BS) >> 6;
      int ids_cur = fetch_ids(l_seq, l_nblk, lw);
      int ids_nxt = fetch_ids(l_seq, l_nblk, lw + 1);
      int ids_row0 = fetch_ids(l_seq, l_nblk, 0);
      int ids_row1 = fetch_ids(l_seq, l_nblk, 1);
      int pf_seq = next_seq(l_seq);
      int pf_nblk = pf_seq < N ? blocks_of(lenf(pf_seq)) : 0;
      int ids_pf0 = pf_seq < N ? fetch_ids(pf_seq, pf_nblk, 0) : 0;
      int ids_pf1 = pf_seq < N ? fetch_ids(pf_seq, pf_nblk, 1) : 0;
      int l_pair = 0, l_count = 0;

      // compute side: q of cc's pair, q of the next pair when lc has fetched it
      int c_pair = 0, c_count = 0, seg_jb = cc.j;
      long long seg_t = t0;
      u32x4 qf[NKC], qf_nxt[NKC];
      int qn_pair = -1;
      load_q(qf, cc.s, cc.kv);
#pragma unroll
      for (int c = 0; c < NKC; ++c) qf_nxt[c] = u32x4{0, 0, 0, 0};

      float m = kNegBig;
      float l = 0.f;
      // P.V accumulators.  Vector ALU: acc[h][e] = head h, element col*VE + e, over
      // this lane's tokens.  Matrix cores (MPV): oacc[i][r] = head col, element
      // (4*grp + r)*VE + i, over all tokens.
      constexpr bool MPV = kMatrixPV<DT, GP>;
      float acc[MPV ? 1 : GP][VE];
      f32x4 oacc[MPV ? VE : 1];
#pragma unroll
      for (int h = 0; h < (MPV ? 1 : GP); ++h)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[h][e] = 0.f;
#pragma unroll
      for (int i = 0; i < (MPV ? VE : 1); ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

      // Issue the loads of lc's tile, then step lc (the chunk's last tile is
      // loaded again rather than stepping past it).  A token index past the pair's
      // last token is clamped to it, so every load reads a real row of the
      // sequence; such tokens get weight exactly 0 from the score mask.
      auto load_next = [&](Tile& Tl) __attribute__((always_inline)) {
        const int blk = kTileTokens * lc.j / BS;  // first block of the tile
        if ((blk >> 6) != lw) {                    // a window holds >= 32 tiles
          ++lw;
          ids_cur = ids_nxt;
          ids_nxt = fetch_ids(l_seq, l_nblk, lw + 1);
        }
        const int a = kTileTokens * lc.j;
        int last = lc.L - 1;
        const int raw0 = __builtin_amdgcn_readlane(ids_cur, blk & 63);
        if constexpr (ROWS) {
          // shared-prefix tables: tokens past the end of the tile's region (a member's
          // padding, whose slots need not hold finite values) read its last token instead
          Tl.vis = raw0;
          if (p.shared)
            last = min(last, blk * BS + (int)(((unsigned)raw0 >> kSharedEndShift) & 31u));
        }
        const int tk = min(a + col, last);
        int tv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) tv[j] = min(a + 4 * grp + j, last);
        int pk, pv[4];
        if constexpr (BS == 8) {
          // a tile spans two blocks; it starts on a multiple of 16 tokens
          const int ida = valid_id(ROWS ? raw0 & id_mask : raw0);
          const int idb = valid_id(ROWS ? __builtin_amdgcn_readlane(ids_cur, (blk & 63) + 1) & id_mask
                                        : __builtin_amdgcn_readlane(ids_cur, (blk & 63) + 1));
          pk = (tk & 8) ? idb : ida;
#pragma unroll
          for (int j = 0; j < 4; ++j) pv[j] = (tv[j] & 8) ? idb : ida;
        } else {
          const int id = valid_id(ROWS ? raw0 & id_mask : raw0);
          pk = id;
#pragma unroll
          for (int j = 0; j < 4; ++j) pv[j] = id;
        }
        const char* kp = (const char*)p.k_cache + (size_t)lc.kv * ROWB + (size_t)pk * blk_bytes +
                         (size_t)(tk % BS) * tok_stride;
        const char* vb = (const char*)p.v_cache + (size_t)lc.kv * ROWB + col * (VE * EB);
        if constexpr (APPEND) {
          // In the pair's last tile the newest token is read from the appended rows (the
          // merge kernel, which runs after this one, stores them into their slot).  The
          // addresses are selected without a branch.
          const bool newest = lc.j + 1 == lc.n;
          const size_t nrow = ((size_t)lc.s * Hkv + lc.kv) * ROWB;
          const char* nv = (const char*)p.new_v + nrow + col * (VE * EB);
          kp = newest && tk == last ? (const char*)p.new_k + nrow : kp;
#pragma unroll
          for (int c = 0; c < NKC; ++c) Tl.k[c] = load16_kv<STREAM>(kp + (4 * c + grp) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const char* vp = vb + (size_t)pv[j] * blk_bytes + (size_t)(tv[j] % BS) * tok_stride;
            load_dwords<STREAM, VW>(newest && tv[j] == last ? nv : vp, Tl.v[j]);
          }
        } else {
#pragma unroll
          for (int c = 0; c < NKC; ++c) Tl.k[c] = load16_kv<STREAM>(kp + (4 * c + grp) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            load_dwords<STREAM, VW>(vb + (size_t)pv[j] * blk_bytes + (size_t)(tv[j] % BS) * tok_stride, Tl.v[j]);
        }

        TileCursor nx = lc;  // a chunk never ends past the batch, so the step succeeds
        if (l_count + 1 < nt && nx.next(N, Hkv, lenf)) {
          ++l_count;
          const int old_s = lc.s, old_kv = lc.kv;
          lc = nx;
          if (lc.s != old_s || lc.kv != old_kv) {  // lc entered the next pair
            ++l_pair;
            if (lc.s != old_s) {
              l_seq = lc.s;
              l_nblk = blocks_of(lc.L);
              if (pf_seq == l_seq) {
                ids_row0 = ids_pf0;
                ids_row1 = ids_pf1;
              } else {
                ids_row0 = fetch_ids(l_seq, l_nblk, 0);
                ids_row1 = fetch_ids(l_seq, l_nblk, 1);
              }
              pf_seq = next_seq(l_seq);
              pf_nblk = pf_seq < N ? blocks_of(lenf(pf_seq)) : 0;
              ids_pf0 = pf_seq < N ? fetch_ids(pf_seq, pf_nblk, 0) : 0;
              ids_pf1 = pf_seq < N ? fetch_ids(pf_seq, pf_nblk, 1) : 0;
            }
            lw = 0;
            ids_cur = ids_row0;
            ids_nxt = ids_row1;
            if (l_pair == c_pair + 1) {
              load_q(qf_nxt, lc.s, lc.kv);
              qn_pair = l_pair;
            }
          }
        }
      };

      // Record a finished piece of a split pair: owner bookkeeping shared by both
      // accumulator layouts.
      auto note_piece = [&](int s, int kv, int jb, int n_pair, long long tseg) __attribute__((always_inline)) {
        if (jb == 0) {
          meta_s = s;
          meta_kv = kv;
          meta_parts = (int)(plan.chunk_of(tseg + n_pair - 1) - ck + 1);
        } else {
          meta_first = 1;
        }
      };

      // Matrix-core layout: every row group already holds the full sums of head col
      // for its 4*VE elements, and the reference maximum m is the same in all four
      // groups; only the running sums are added over the groups.
      // ROWS: store one piece's partial result (running max, sum and unnormalised
      // accumulator of every row) in its slot.  The slot holds R rows x D floats in 16-byte
      // chunks: chunk j of lane (grp, col), elements (4 grp + r) VE + i .. + 3 of row col
      // with j = r VE/4 + i/4, sits at chunk (4 j + grp) R + col, so each store instruction
      // writes 4 R consecutive chunks (whole cache lines) and the merge reads them back the
      // same way.  The decode variants keep row-major slots.
      auto store_piece = [&](size_t slot, const f32x4 (&acc4)[MPV ? VE : 1], float mx, float sum, int R)
          __attribute__((always_inline)) {
        f32x4* dst = reinterpret_cast<f32x4*>(p.ws_acc + slot * R * D);
        const int off0 = grp * R + col, stride = 4 * R;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < VE; i += 4)
            dst[off0 + (r * (VE / 4) + i / 4) * stride] =
                f32x4{acc4[i][r], acc4[i + 1][r], acc4[i + 2][r], acc4[i + 3][r]};
        if (grp == 0) {
          float* ml = p.ws_ml + (slot * R + col) * 2;
          ml[0] = mx;
          ml[1] = sum;
        }
      };
      // Matrix-core P.V: a chunk's first piece, when the chunk goes on past it, is kept in
      // registers and stored after the chunk's last tile, so that no load wait inside the
      // stream also waits for those stores (stores and loads share one counter).
      // Llama-3-8B decode 389.6 against 394 us; verification 411 against 446.
      f32x4 def_acc[MPV ? VE : 1];
      float def_m = 0.f, def_l = 0.f;
      size_t def_slot = 0;
      bool has_def = false;

      auto flush_mpv = [&](int s, int kv, int jb, int je, int L, long long tseg, bool chunk_end) __attribute__((always_inline)) {
        float ls = l;
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        const int n_pair = tiles_of(L);
        const int d0 = 4 * grp * VE;  // first element of this lane's run
        const int R = ROWS ? p.rows : g;
        if (col < R) {
          float o[4 * VE];
          if (jb == 0 && je == n_pair) {
            size_t orow = (size_t)s * p.num_heads + kv * g + col;
            bool out_ok = true;
            if constexpr (ROWS) {
              // (a row that saw no token, an empty member of a shared-prefix group, keeps
              // the zeros the layout kernel wrote)
              const int q0 = qsf(s);
              out_ok = row_i < qsf(s + 1) - q0 && ls != 0.f;
              orow = (size_t)(q0 + row_i) * p.num_heads + kv * g + row_h;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int i = 0; i < VE; ++i) o[r * VE + i] = oacc[i][r] / ls;
            if (out_ok) store_row<DT, 4 * VE>((char*)p.out + orow * ROWB + d0 * EB, o);
          } else {
            const size_t slot = 2 * (size_t)ck + (jb == 0 ? 1 : 0);
            if (jb != 0 && !chunk_end) {
#pragma unroll
              for (int i = 0; i < (MPV ? VE : 1); ++i) def_acc[i] = oacc[i];
              def_m = m;
              def_l = ls;
              def_slot = slot;
            } else if constexpr (ROWS) {
              store_piece(slot, oacc, m, ls, R);
            } else {
              // row-major slots: row col's elements d0 .. d0 + 4 VE - 1 from this lane
              float* dst = p.ws_acc + (slot * R + col) * D + d0;
#pragma unroll
              for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < VE; i += 4)
                  *reinterpret_cast<f32x4*>(dst + r * VE + i) =
                      f32x4{oacc[i][r], oacc[i + 1][r], oacc[i + 2][r], oacc[i + 3][r]};
              if (grp == 0) {
                float* ml = p.ws_ml + (slot * R + col) * 2;
                ml[0] = m;
                ml[1] = ls;
              }
            }
          }
        }
        if (jb != 0 && !chunk_end) has_def = true;
        if (!(jb == 0 && je == n_pair)) note_piece(s, kv, jb, n_pair, tseg);
        m = kNegBig;
        l = 0.f;
#pragma unroll
        for (int i = 0; i < VE; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      };

      // Normalise or store the finished segment [jb, je) of pair (s, kv).
      auto flush = [&](int s, int kv, int jb, int je, int L, long long tseg, bool chunk_end) __attribute__((always_inline)) {
        if constexpr (MPV) {
          flush_mpv(s, kv, jb, je, L, tseg, chunk_end);
        } else {
          // Merge the four per-group streams of every head.
          float M = fmaxf(m, __shfl_xor(m, 16));
          M = fmaxf(M, __shfl_xor(M, 32));
          const float f = fast_exp2(m - M);
          float ls = l * f;
          ls += __shfl_xor(ls, 16);
          ls += __shfl_xor(ls, 32);
          static_for<GP>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const float fh = row_bcast<h>(f);
#pragma unroll
            for (int e = 0; e < VE; ++e) {
              float x = acc[h][e] * fh;
              x += __shfl_xor(x, 16);
              x += __shfl_xor(x, 32);
              acc[h][e] = x;
            }
          });
          const int head0 = kv * g;
          const int n_pair = tiles_of(L);
          if (jb == 0 && je == n_pair) {
            // whole pair in this chunk: every row now holds the full sums; row grp
            // stores heads h = grp (mod 4)
            static_for<GP>([&](auto hc) {
              constexpr int h = decltype(hc)::value;
              const float lh = row_bcast<h>(ls);
              if (h < g && (h & 3) == grp) {
                float o[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e) o[e] = acc[h][e] / lh;
                store_row<DT, VE>((char*)p.out + ((size_t)s * p.num_heads + head0 + h) * ROWB + col * (VE * EB), o);
              }
            });
          } else {
            // one piece of a pair split over chunks: the owner (first tile) writes to
            // slot 2c + 1, every other piece is its chunk's first segment, slot 2c
            const bool owner = jb == 0;
            const size_t slot = 2 * (size_t)ck + (owner ? 1 : 0);
            static_for<GP>([&](auto hc) {
              constexpr int h = decltype(hc)::value;
              if (h < g && (h & 3) == grp) {
                float* dst = p.ws_acc + (slot * g + h) * D + col * VE;
#pragma unroll
                for (int e = 0; e < VE; e += 4)
                  *reinterpret_cast<f32x4*>(dst + e) = f32x4{acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]};
              }
            });
            if (grp == 0 && col < g) {
              float* ml = p.ws_ml + (slot * g + col) * 2;
              ml[0] = M;
              ml[1] = ls;
            }
            note_piece(s, kv, jb, n_pair, tseg);
          }
          m = kNegBig;
          l = 0.f;
#pragma unroll
          for (int h = 0; h < (MPV ? 1 : GP); ++h)
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[h][e] = 0.f;
        }
      };

      // Fold cc's tile into the running softmax, flush at the end of a segment,
      // then step cc.
      auto compute_next = [&](const Tile& Tl) __attribute__((always_inline)) {
        // S = K q^T on the matrix cores
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
          if constexpr (DT == kBF16) {
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Tl.k[c]),
                                                         __builtin_bit_cast(bf16x8, qf[c]), sc, 0, 0, 0);
          } else if constexpr (DT == kF16) {
            sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, Tl.k[c]),
                                                        __builtin_bit_cast(f16x8, qf[c]), sc, 0, 0, 0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(Tl.k[c][e]),
                                                        __uint_as_float(qf[c][e]), sc, 0, 0, 0);
          }
        }
        // online softmax, stream (grp, head col); tokens past the end get -inf
        int lim;
        if constexpr (ROWS) {
          if (p.shared) {
            // the tile's owner and the tokens of its region from the tile's start
            const unsigned u = (unsigned)Tl.vis;
            const int own = (int)(u >> kSharedOwnerShift);
            const int cnt = (int)((u >> kSharedEndShift) & 31u) + 1 - (kTileTokens * cc.j) % BS;
            lim = own == kSharedAll || own == c_vis ? cnt - 4 * grp : 0;
          } else {
            lim = c_vis - kTileTokens * cc.j - 4 * grp;
          }
        } else {
          lim = cc.L - kTileTokens * cc.j - 4 * grp;
        }
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[r] = r < lim ? sc[r] * sl2 : -__builtin_inff();
        if constexpr (MPV) {
          // One reference maximum per head for all 16 tokens (the product below sums
          // over every row group), moved only when the tile exceeds it by kLazyMax.
          const float tmx = max_over_rows(fmaxf(fmaxf(fmaxf(sv[0], sv[1]), sv[2]), sv[3]));
          if (__any(tmx > m + kLazyMax)) {
            const float mn = tmx > m + kLazyMax ? tmx : m;
            const float alpha = fast_exp2(m - mn);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < VE; ++i) oacc[i] *= alpha;
            m = mn;
          }
          float pr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sv[r] - m);
          // P^T as the B operand (tokens 4*grp + r of head col).  bf16 keeps 8
          // significant bits, so P is split in two: the high term is P cut to its top
          // 16 bits (the remainder is exact in fp32) and the low term that remainder
          // rounded; the running sum adds the fp32 weights.  fp16 keeps 11 bits in one
          // term and the running sum adds the rounded weights.
          uint32_t ph[2], pl[2];
          if constexpr (DT == kBF16) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const uint32_t x = __float_as_uint(pr[2 * u]), y = __float_as_uint(pr[2 * u + 1]);
              ph[u] = (x >> 16) | (y & 0xffff0000u);
              pl[u] = pack2<DT>(pr[2 * u] - __uint_as_float(x & 0xffff0000u),
                                pr[2 * u + 1] - __uint_as_float(y & 0xffff0000u));
            }
            l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
          } else {
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              ph[u] = pack2<DT>(pr[2 * u], pr[2 * u + 1]);
              const f16x2 h = __builtin_bit_cast(f16x2, ph[u]);
              ps += (float)h.x + (float)h.y;
              pl[u] = 0u;
            }
            l += ps;
          }
          // O^T += V^T P^T: the A operand of product i is element col*VE + i of the
          // lane's four token rows (row m = col of the 16x16 tile), so the result row
          // 4*grp + r stands for element (4*grp + r)*VE + i.
#pragma unroll
          for (int i = 0; i < VE; ++i) {
            const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t a0 = __builtin_amdgcn_perm(Tl.v[1][i >> 1], Tl.v[0][i >> 1], sel);
            const uint32_t a1 = __builtin_amdgcn_perm(Tl.v[3][i >> 1], Tl.v[2][i >> 1], sel);
            oacc[i] = mfma16<DT>(a0, a1, ph[0], ph[1], oacc[i]);
            if constexpr (DT == kBF16) oacc[i] = mfma16<DT>(a0, a1, pl[0], pl[1], oacc[i]);
          }
        } else {
          const float mn = fmaxf(fmaxf(fmaxf(fmaxf(m, sv[0]), sv[1]), sv[2]), sv[3]);
          const float alpha = fast_exp2(m - mn);
          float pr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sv[r] - mn);
          l = l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
          m = mn;
          // rescale the accumulators only when some running max moved
          if (__any(col < GP && alpha != 1.0f)) {
            static_for<GP>([&](auto hc) {
              constexpr int h = decltype(hc)::value;
              const float a = row_bcast<h>(alpha);
#pragma unroll
              for (int e = 0; e < VE; ++e) acc[h][e] *= a;
            });
          }
          // P V on the vector ALU
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float vf[VE];
            unpack<DT, VW>(Tl.v[j], vf);
            static_for<GP>([&](auto hc) {
              constexpr int h = decltype(hc)::value;
              const float pj = row_bcast<h>(pr[j]);
#pragma unroll
              for (int e = 0; e < VE; ++e) acc[h][e] = fmaf(pj, vf[e], acc[h][e]);
            });
          }
        }

        TileCursor nx = cc;  // as for lc, the step succeeds whenever a tile is left
        const bool last_tile = c_count + 1 == nt || !nx.next(N, Hkv, lenf);
        if (last_tile || cc.j + 1 == cc.n) {
          flush(cc.s, cc.kv, seg_jb, cc.j + 1, cc.L, seg_t, last_tile);
          if (!last_tile) {  // on to the next pair
            cc = nx;
            if constexpr (ROWS) c_vis = visible(cc.s, cc.L);
            ++c_count;
            ++c_pair;
            seg_jb = 0;
            seg_t = t0 + c_count;
            if (qn_pair == c_pair) {
#pragma unroll
              for (int c = 0; c < NKC; ++c) qf[c] = qf_nxt[c];
            } else {
              load_q(qf, cc.s, cc.kv);
            }
          }
        } else {
          cc = nx;
          ++c_count;
        }
      };

      // kDecodePipe tiles in flight: while one is reduced the next ones are being
      // fetched.  Loads are unconditional so no tile register is ever copied, and
      // the scheduling barriers keep a refill after the last use of the registers
      // it overwrites.
      Tile tl[kDecodePipe];
      static_for<kDecodePipe>([&](auto ic) {
        load_next(tl[decltype(ic)::value]);
        __builtin_amdgcn_sched_barrier(0);
      });
      for (int tt = 0; tt < nt; tt += kDecodePipe) {
        static_for<kDecodePipe>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if (i == 0 || tt + i < nt) compute_next(tl[i]);
          __builtin_amdgcn_sched_barrier(0);
          load_next(tl[i]);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      if constexpr (ROWS) {
        if (has_def && col < p.rows) store_piece(def_slot, def_acc, def_m, def_l, p.rows);
      } else if constexpr (MPV) {
        if (has_def && col < g) {
          float* dst = p.ws_acc + (def_slot * g + col) * D + 4 * grp * VE;
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < VE; i += 4)
              *reinterpret_cast<f32x4*>(dst + r * VE + i) =
                  f32x4{def_acc[i][r], def_acc[i + 1][r], def_acc[i + 2][r], def_acc[i + 3][r]};
          if (grp == 0) {
            float* ml = p.ws_ml + (def_slot * g + col) * 2;
            ml[0] = def_m;
            ml[1] = def_l;
          }
        }
      }
    }
    // Every chunk states whether it owns a split pair (parts >= 2) and whether it
    // left a first piece of one in slot 2c.
    if (lane == 0)
      *reinterpret_cast<u32x4*>(chunk_meta + 4 * ck) =
          u32x4{(uint32_t)meta_s, (uint32_t)meta_kv, (uint32_t)meta_parts, (uint32_t)meta_first};
  }
}

// Merge the pieces of every pair split over chunks, and hand the workspace back
// ready for the next call (tail counter at 0).  Wave k of workgroup b handles the
// pair owned by chunk c = 4 b + k, if any, all query heads of the group at once
// (64 / GP lanes per head).  The pieces are the owner's (slot 2c + 1) and the
// first piece of every later chunk up to the pair's last one that left one (slot
// 2c'); empty tail chunks leave none.  They are folded in chunk order with the
// same running-max rule as the blocks of one piece:
//     m' = max(m, m_i),  l' = 2^(m - m') l + 2^(m_i - m') l_i,
//     acc' = 2^(m - m') acc + 2^(m_i - m') a_i,      out = acc / l,
// so the result does not depend on timing.
//
// For pa_decode_append the workgroups from merge_blocks on store each sequence's
// newest K and V rows (read from new_k/new_v by the decode kernel, which has
// finished) into the slot of position L - 1, 16 bytes per lane, alongside the merges.
template <int DT, int D, int GP, bool ROWS>
__global__ __launch_bounds__(256) void reduce_kernel(DecodeParams p) {
  constexpr int LPH = 64 / GP;   // lanes per head
  constexpr int EPL = D / LPH;   // accumulator elements per lane
  constexpr int EB = Elem<DT>::bytes;
  static_assert(!ROWS || (kMatrixPV<DT, GP> && EPL % 4 == 0), "chunked slots hold 4-element runs");
  if ((int)blockIdx.x >= p.merge_blocks) {
    constexpr int PPR = D * EB / 16;  // 16-byte pieces per row
    const long long x = (long long)(blockIdx.x - p.merge_blocks) * 256 + threadIdx.x;
    if (x >= (long long)p.num_seqs * p.num_kv_heads * PPR) return;
    const long long row = x / PPR;  // row (s, kv) of new_k and new_v
    const int piece = (int)(x % PPR);
    const int s = (int)(row / p.num_kv_heads);
    const int kv = (int)(row % p.num_kv_heads);
    const int L = seq_len_at(p, s);
    if (L == 0) return;
    const int id = p.block_tables[(size_t)s * p.max_blocks_per_seq + (L - 1) / p.block_size];
    if ((unsigned)id >= (unsigned)p.num_blocks) return;  // contract violation: no write
    const size_t slot = (size_t)id * p.block_size + (L - 1) % p.block_size;
    const size_t dst = (slot * p.num_kv_heads + kv) * (D * EB) + piece * 16;
    const size_t src = (size_t)row * (D * EB) + piece * 16;
    const u32x4 k = *reinterpret_cast<const u32x4*>((const char*)p.new_k + src);
    const u32x4 v = *reinterpret_cast<const u32x4*>((const char*)p.new_v + src);
    *reinterpret_cast<u32x4*>((char*)p.k_cache + dst) = k;
    *reinterpret_cast<u32x4*>((char*)p.v_cache + dst) = v;
    return;
  }
  int* const hdr = p.ws_meta;
  const int* const chunk_meta = p.ws_meta + 64;
  if (blockIdx.x == 0 && threadIdx.x == 0) hdr[32] = 0;
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nchunks = hdr[0];
  if (c >= nchunks) return;
  // A chunk record is written by the chunk's wave in this call; the checks keep a
  // stale record (a workspace never zeroed, whose counter handed out no tail) inside
  // the chunk list and the output.
  const int* meta = chunk_meta + 4 * (size_t)c;
  // the "left a first piece" flags of the next 63 chunks load together with the record
  // (only those below c + parts are used)
  const int flag1 = lane >= 1 && c + lane < nchunks ? chunk_meta[4 * ((size_t)c + lane) + 3] : 0;
  const int parts = min(meta[2], nchunks - c);
  if (parts < 2) return;
  const int s = meta[0];
  const int kv = meta[1];
  if (s < 0 || s >= p.num_seqs || kv < 0 || kv >= p.num_kv_heads) return;
  const int g = p.group;
  const int R = p.rows;          // rows of a pair: the group's heads, or (query, head) rows
  const int h = lane / LPH;
  const int sub = lane % LPH;
  const int hr = h < R ? h : 0;  // lanes of padding rows read row 0 and store nothing

  float m = kNegBig, l = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  // Piece i of the pair: i = 0 is the owner's (slot 2c + 1), i >= 1 the first piece of
  // chunk c + i (slot 2(c + i)) if that chunk left one.  The flags of 64 chunks are read
  // at once, and the pieces are loaded in batches (8, or 4 for the widest rows) before
  // they are folded, so a pair cut into many pieces costs a few dependent loads, not two
  // per piece.  The fold order is the chunk order.
  constexpr int kBatch = EPL <= 16 ? 8 : 4;
  for (int i0 = 0; i0 < parts; i0 += 64) {
    const int i = i0 + lane;
    const int flag = i0 == 0 ? flag1 : (i < parts ? chunk_meta[4 * ((size_t)c + i) + 3] : 0);
    unsigned long long has = __ballot(i < parts && (i == 0 || flag != 0));
    while (has) {
      int bi[kBatch];
      bool ok[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        ok[k] = has != 0;
        bi[k] = ok[k] ? i0 + __ffsll(has) - 1 : 0;
        has &= has - 1;
      }
      float mi[kBatch], li[kBatch], av[kBatch][EPL];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (!ok[k]) continue;
        const size_t sl = bi[k] == 0 ? 2 * (size_t)c + 1 : 2 * ((size_t)c + bi[k]);
        const size_t r = sl * R + hr;
        mi[k] = p.ws_ml[2 * r];
        li[k] = p.ws_ml[2 * r + 1];
        if constexpr (ROWS) {
          // the rows mode's chunked slot layout (store_piece): element e = (4 grp + r) VE + i
          // of row hr is in chunk (4 (r VE/4 + i/4) + grp) R + hr
          constexpr int VE = D / 16;
          const f32x4* a = reinterpret_cast<const f32x4*>(p.ws_acc + sl * R * D);
#pragma unroll
          for (int e4 = 0; e4 < EPL; e4 += 4) {
            const int e = sub * EPL + e4;
            const int grp = e / (4 * VE), rr = (e / VE) % 4, i = e % VE;
            const f32x4 x = a[(4 * (rr * (VE / 4) + i / 4) + grp) * R + hr];
            av[k][e4] = x[0];
            av[k][e4 + 1] = x[1];
            av[k][e4 + 2] = x[2];
            av[k][e4 + 3] = x[3];
          }
        } else {
          const float* a = p.ws_acc + r * D + sub * EPL;
#pragma unroll
          for (int e = 0; e < EPL; ++e) av[k][e] = a[e];
        }
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (!ok[k]) continue;
        const float mn = fmaxf(m, mi[k]);
        const float fa = fast_exp2(m - mn);
        const float fb = fast_exp2(mi[k] - mn);
        l = fmaf(li[k], fb, l * fa);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(av[k][e], fb, acc[e] * fa);
        m = mn;
      }
    }
  }
  size_t orow = (size_t)s * p.num_heads + kv * g + h;
  bool ok = h < R;
  if constexpr (ROWS) {  // row h is query h / g, head h % g
    const int q0 = min(max(p.q_start[s], 0), p.total_q);
    const int i = h / g;
    ok = ok && i < min(max(p.q_start[s + 1], 0), p.total_q) - q0 && l != 0.f;
    orow = (size_t)(q0 + i) * p.num_heads + kv * g + (h - i * g);
  }
  if (ok) {
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = acc[e] / l;
    store_row<DT, EPL>((char*)p.out + orow * (D * EB) + sub * (EPL * EB), o);
  }
}

// The decode and merge kernels of one shape (false if not compiled).  Four decode
// variants: streaming K/V loads (pa_decode), the same with the append
// (pa_decode_append), default-policy loads (pa_decode_cached), and the multi-query rows
// (pa_multi_query with at most 16 rows per (sequence, KV head), 16-bit types, GP = 16).
template <int DT, int D, int BS, int GP>
bool pick(DecodeVariant v, const void** dec, const void** red) {
  switch (v) {
    case DecodeVariant::kStream: *dec = reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, GP, false, true, false>); break;
    case DecodeVariant::kAppend: *dec = reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, GP, true, true, false>); break;
    case DecodeVariant::kCached: *dec = reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, GP, false, false, false>); break;
    case DecodeVariant::kRows:
      if constexpr (GP == 16 && DT != kF32) {
        *dec = reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, GP, false, true, true>);
        break;
      } else {
        return false;
      }
    default: return false;
  }
  *red = v == DecodeVariant::kRows ? reinterpret_cast<const void*>(&reduce_kernel<DT, D, GP, GP == 16 && DT != kF32>)
                                   : reinterpret_cast<const void*>(&reduce_kernel<DT, D, GP, false>);
  return true;
}

template <int DT, int D, int BS>
bool pick_group(int gp, DecodeVariant variant, const void** dec, const void** red) {
  switch (gp) {
    case 1: return pick<DT, D, BS, 1>(variant, dec, red);
    case 2: return pick<DT, D, BS, 2>(variant, dec, red);
    case 4: return pick<DT, D, BS, 4>(variant, dec, red);
    case 8: return pick<DT, D, BS, 8>(variant, dec, red);
    case 16: return pick<DT, D, BS, 16>(variant, dec, red);
    default: return false;
  }
}

template <int DT, int D>
bool pick_block(int bs, int gp, DecodeVariant variant, const void** dec, const void** red) {
  switch (bs) {
    case 8: return pick_group<DT, D, 8>(gp, variant, dec, red);
    case 16: return pick_group<DT, D, 16>(gp, variant, dec, red);
    case 32: return pick_group<DT, D, 32>(gp, variant, dec, red);
    default: return false;
  }
}

template <int DT>
bool pick_decode_kernels(int head_dim, int bs, int gp, DecodeVariant variant, const void** dec, const void** red) {
  switch (head_dim) {
    case 64: return pick_block<DT, 64>(bs, gp, variant, dec, red);
    case 128: return pick_block<DT, 128>(bs, gp, variant, dec, red);
    default: return false;
  }
}

}  // namespace pagedkv
