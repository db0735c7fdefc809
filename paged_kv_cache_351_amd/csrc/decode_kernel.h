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
//   every one of the launched waves (one 64-lane wave per workgroup, as many as
//   the chip holds at once) takes the same number of consecutive tiles.  Each
//   wave therefore reads the same number of K/V bytes whatever the length mix,
//   and no wave waits for a second round of dispatch.  A pair that falls entirely
//   inside one wave is finished there; a pair cut by a wave boundary leaves one
//   partial result per piece, and reduce_kernel merges them.  Every query head of
//   a KV head's group (g = num_heads / num_kv_heads <= GP) is handled by the same
//   wave, so each K/V row is read from HBM once.
//
// Prologue
//   Each wave sums the tile counts of all sequences (64 at a time, one per lane)
//   to get the total T, and scans them again to find the pair and tile where its
//   range begins.  Sequences of length 0 have no tiles; their zero outputs are
//   written by wave s mod (number of waves).
//
// Lane roles inside a segment (lane = 16 * grp + col, grp = 0..3, col = 0..15)
//   q.K^T on the matrix cores: v_mfma_f32_16x16x32_{bf16,f16} (or 16x16x4_f32)
//     with A = the tile's K rows (row = token col, this lane's 16-byte chunks
//     4c + grp of the row) and B = the group's query rows padded to 16 columns
//     (column = head col, same chunks).  Any fixed assignment of head_dim
//     positions to MFMA k-slots gives the same dot products, so the chunking
//     only has to match between A and B.  The result lands as
//     S[token 4*grp + r][head col], r = 0..3, in lane (grp, col).
//   Online softmax: lane (grp, col) keeps its own running max m and sum l for
//     head col over the tokens 4*grp + r of every tile, i.e. four independent
//     streams per head; they are merged once at the end of the segment.
//   P.V on the vector ALU: lane (grp, col) owns head_dim/16 consecutive
//     elements (at col * head_dim/16) of tokens 4*grp + j, j = 0..3, and
//     accumulates acc[h][.] for every head h of the group.  The weight p of
//     (head h, token 4*grp + j) sits in lane (grp, h); DPP row_newbcast:h
//     broadcasts it to the 16 lanes of the row -- no LDS, no barrier.
//   Block ids: a segment is walked in windows of up to 64 blocks; lane i holds
//     the id of the window's block i (v_readlane picks it per tile), and the next
//     window's ids are fetched while the current one is processed.
//
// Logits are taken in base 2 (scale * log2 e folded in), so every exponential is
// one v_exp_f32.  Running maxima start at a finite -1e30 so that a stream with
// no valid token yet never forms inf - inf.  Tokens past the end of a window in
// its last tile are redirected to the window's last token before loading (so no
// unused slot is ever read) and their scores are replaced by -inf with a select,
// which makes their weights exactly 0.
#pragma once

#include <type_traits>

#include "common.h"
#include "split.h"

namespace pagedkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;

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

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
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
    if constexpr (N == 8) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    } else if constexpr (N == 4) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
    } else if constexpr (N == 2) {
      *reinterpret_cast<uint32_t*>(dst) = w[0];
    } else {
      static_assert(N == 1, "row piece of 1, 2, 4 or 8 elements");
      if constexpr (DT == kBF16) *reinterpret_cast<__bf16*>(dst) = (__bf16)v[0];
      else *reinterpret_cast<_Float16*>(dst) = (_Float16)v[0];
    }
  }
}

template <int NW>
__device__ __forceinline__ void load_dwords(const char* src, uint32_t (&w)[NW]) {
  static_assert(NW == 2 || NW % 4 == 0, "row slice must be 8 or a multiple of 16 bytes");
  if constexpr (NW == 2) {
    u32x2 x = *reinterpret_cast<const u32x2*>(src);
    w[0] = x.x;
    w[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      u32x4 x = reinterpret_cast<const u32x4*>(src)[i];
      w[4 * i] = x.x;
      w[4 * i + 1] = x.y;
      w[4 * i + 2] = x.z;
      w[4 * i + 3] = x.w;
    }
  }
}

template <int DT, int D, int BS, int GP>
__global__ __launch_bounds__(64) void decode_kernel(DecodeParams p) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int ROWB = D * EB;       // bytes of one (token, KV head) row
  constexpr int NKC = ROWB / 64;     // 16-byte K chunks per lane per tile
  constexpr int VE = D / 16;         // V elements per lane per token
  constexpr int VW = VE * EB / 4;    // V dwords per lane per token
  static_assert(ROWB % 64 == 0 && (BS == 8 || BS == 16 || BS == 32), "shape");

  const int lane = threadIdx.x;
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int w = blockIdx.x;
  const int launched = gridDim.x;
  const int N = p.num_seqs;
  const int Hkv = p.num_kv_heads;
  const int g = p.group;

  // Zero outputs of empty sequences.
  for (int s = w; s < N; s += launched) {
    if (seq_len_at(p, s) == 0) {
      u32x4* o = reinterpret_cast<u32x4*>((char*)p.out + (size_t)s * p.num_heads * ROWB);
      const int n16 = p.num_heads * ROWB / 16;
      for (int i = lane; i < n16; i += 64) o[i] = u32x4{0, 0, 0, 0};
    }
  }

  // Total tiles of the step.
  long long seq_tiles = 0;
  for (int c = 0; c < N; c += 64) {
    const int s = c + lane;
    seq_tiles += __builtin_amdgcn_readfirstlane(wave_sum(s < N ? tiles_of(seq_len_at(p, s)) : 0));
  }
  const long long T = seq_tiles * Hkv;
  const long long nw = waves_used(T, launched);

  int meta_s = 0, meta_kv = 0, meta_parts = 0;

  if (w < nw) {
    const long long t0 = wave_begin(w, T, nw);
    const long long t1 = wave_begin(w + 1, T, nw);
    // Find the pair and tile of t0: the first sequence whose tiles end past t0.
    int s0 = -1;
    long long pair_base = 0;
    long long base = 0;
    for (int c = 0; c < N; c += 64) {
      const int s = c + lane;
      const int n = s < N ? tiles_of(seq_len_at(p, s)) : 0;
      const int incl = wave_inclusive_scan(n);
      const unsigned long long hit = __ballot(base + (long long)incl * Hkv > t0);
      if (hit) {
        const int ln = __ffsll(hit) - 1;
        s0 = c + ln;
        pair_base = base + (long long)__builtin_amdgcn_readlane(incl - n, ln) * Hkv;
        break;
      }
      base += (long long)__builtin_amdgcn_readlane(incl, 63) * Hkv;
    }
    // s0 >= 0 always (t0 < T); the test only guards against reading past the lengths
    const int n0 = s0 >= 0 ? tiles_of(seq_len_at(p, s0)) : 0;
    const long long off = t0 - pair_base;
    const int kv0 = n0 > 0 ? (int)(off / n0) : 0;
    const int j0 = n0 > 0 ? (int)(off % n0) : 0;

    const size_t tok_stride = (size_t)Hkv * ROWB;
    const size_t blk_bytes = (size_t)BS * tok_stride;
    const float sl2 = p.scale_log2e;

    long long t_seg = t0;  // global index of the current segment's first tile
    auto segment = [&](int s, int kv, int jb, int je, int L) __attribute__((always_inline)) {
      const int tok0 = jb * kTileTokens;
      const int tok_end = min(je * kTileTokens, L);
      const int head0 = kv * g;
      const char* kbase = (const char*)p.k_cache + (size_t)kv * ROWB;
      const char* vbase = (const char*)p.v_cache + (size_t)kv * ROWB + col * (VE * EB);
      const int* trow = p.block_tables + (size_t)s * p.max_blocks_per_seq;
      const int b_first = tok0 / BS;
      const int b_end = (tok_end + BS - 1) / BS;

      // Query fragments (MFMA B operand): head head0 + col, chunks 4c + grp.
      u32x4 qf[NKC];
      {
        const char* qrow = (const char*)p.q + ((size_t)s * p.num_heads + head0 + col) * ROWB;
#pragma unroll
        for (int c = 0; c < NKC; ++c)
          qf[c] = col < g ? *reinterpret_cast<const u32x4*>(qrow + (4 * c + grp) * 16) : u32x4{0, 0, 0, 0};
      }

      // Block ids of the window starting at block wb, one per lane.  An id outside
      // the pool is a contract violation; it becomes 0 so no access leaves the pool.
      auto load_ids = [&](int wb) __attribute__((always_inline)) {
        int id = 0;
        if (wb + lane < b_end) {
          id = trow[wb + lane];
          id = (unsigned)id < (unsigned)p.num_blocks ? id : 0;
        }
        return id;
      };

      float m = kNegBig;
      float l = 0.f;
      float acc[GP][VE];
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[h][e] = 0.f;

      struct Tile {
        u32x4 k[NKC];
        uint32_t v[4][VW];
      };

      int idw = load_ids(b_first);
      for (int wb = b_first; wb < b_end; wb += 64) {
        int idn = 0;
        if (wb + 64 < b_end) idn = load_ids(wb + 64);
        const int w0 = max(tok0, wb * BS);                      // a multiple of 16
        const int wn = min(tok_end, (wb + 64) * BS) - w0;      // tokens in the window
        const int last = wn - 1;

        // Tile tt covers window tokens [16 tt, 16 tt + 16).  A token index past the
        // window's last token is clamped to it, so every load reads a real row of
        // this sequence; such tokens get weight exactly 0 from the score mask.
        auto load_tile = [&](Tile& Tl, int tt) __attribute__((always_inline)) {
          const int a = w0 + kTileTokens * tt;                  // first token of the tile
          const int tk = w0 + min(kTileTokens * tt + col, last);
          int tv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) tv[j] = w0 + min(kTileTokens * tt + 4 * grp + j, last);
          int pk, pv[4];
          if constexpr (BS == 8) {
            const int bi = a / BS - wb;
            const int ida = __builtin_amdgcn_readlane(idw, bi);
            const int idb = __builtin_amdgcn_readlane(idw, bi + 1);
            pk = (tk & 8) ? idb : ida;
#pragma unroll
            for (int j = 0; j < 4; ++j) pv[j] = (tv[j] & 8) ? idb : ida;
          } else {
            const int id = __builtin_amdgcn_readlane(idw, a / BS - wb);
            pk = id;
#pragma unroll
            for (int j = 0; j < 4; ++j) pv[j] = id;
          }
          const char* kp = kbase + (size_t)pk * blk_bytes + (size_t)(tk % BS) * tok_stride;
#pragma unroll
          for (int c = 0; c < NKC; ++c) Tl.k[c] = *reinterpret_cast<const u32x4*>(kp + (4 * c + grp) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            load_dwords<VW>(vbase + (size_t)pv[j] * blk_bytes + (size_t)(tv[j] % BS) * tok_stride, Tl.v[j]);
        };

        auto compute = [&](const Tile& Tl, int tt) __attribute__((always_inline)) {
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
          const int lim = wn - kTileTokens * tt - 4 * grp;
          float sv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[r] = r < lim ? sc[r] * sl2 : -__builtin_inff();
          const float mn = fmaxf(m, fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
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
        };

        // Two tiles in flight: while one is reduced the next two are being fetched.
        // Loads are unconditional (clamped tile index) so no tile register is ever
        // copied, and the scheduling barriers keep a refill after the last use of
        // the registers it overwrites.
        const int n_tiles = (wn + kTileTokens - 1) / kTileTokens;
        const int lt = n_tiles - 1;
        Tile A, B;
        load_tile(A, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_tile(B, min(1, lt));
        __builtin_amdgcn_sched_barrier(0);
        for (int tt = 0; tt < n_tiles; tt += 2) {
          compute(A, tt);
          __builtin_amdgcn_sched_barrier(0);
          load_tile(A, min(tt + 2, lt));
          __builtin_amdgcn_sched_barrier(0);
          if (tt + 1 < n_tiles) compute(B, tt + 1);
          __builtin_amdgcn_sched_barrier(0);
          load_tile(B, min(tt + 3, lt));
          __builtin_amdgcn_sched_barrier(0);
        }
        idw = idn;
      }

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

      const int n_pair = tiles_of(L);
      if (jb == 0 && je == n_pair) {
        // whole pair in this wave: every row now holds the full sums; row grp
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
        // one piece of a pair split over waves: the owner (first tile) writes to
        // slot 2w + 1, every other piece is its wave's first segment, slot 2w
        const bool owner = jb == 0;
        const size_t slot = 2 * (size_t)w + (owner ? 1 : 0);
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
        if (owner) {
          meta_s = s;
          meta_kv = kv;
          meta_parts = (int)(wave_of(t_seg + n_pair - 1, T, nw) - w + 1);
        }
      }
      t_seg += je - jb;
    };

    if (n0 > 0)
      walk_tiles(t0, t1, s0, kv0, j0, N, Hkv, [&](int s) { return seq_len_at(p, s); }, segment);
  }

  // Every launched wave states whether it owns a split pair (parts >= 2).
  if (lane == 0) {
    int* meta = p.ws_meta + 4 * (size_t)w;
    *reinterpret_cast<u32x4*>(meta) = u32x4{(uint32_t)meta_s, (uint32_t)meta_kv, (uint32_t)meta_parts, 0u};
  }
}

// Merge the pieces of every pair split over waves.  Workgroup (w, h) handles query
// head h of the group of the pair wave w owns, if any: with the pieces' running
// maxima m_i, sums l_i and accumulators a_i, M = max_i m_i and
//     out = sum_i 2^(m_i - M) a_i / sum_i 2^(m_i - M) l_i.
// Wave k of the workgroup sums the pieces i = k (mod 4); the four sums are then
// added in a fixed order, so the result does not depend on timing.
template <int DT, int D>
__global__ __launch_bounds__(256) void reduce_kernel(DecodeParams p) {
  constexpr int EPT = D / 64;
  constexpr int EB = Elem<DT>::bytes;
  const int w = blockIdx.x;
  const int h = blockIdx.y;
  const int* meta = p.ws_meta + 4 * (size_t)w;
  const int parts = meta[2];
  if (parts < 2) return;
  const int s = meta[0];
  const int kv = meta[1];
  const int g = p.group;
  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int lane = tid & 63;
  auto slot = [&](int i) -> size_t { return i == 0 ? 2 * (size_t)w + 1 : 2 * ((size_t)w + i); };

  __shared__ float red_max[4];
  __shared__ float red_l[4];
  __shared__ float red_acc[4][D];

  float mx = kNegBig;
  for (int i = tid; i < parts; i += 256) mx = fmaxf(mx, p.ws_ml[(slot(i) * g + h) * 2]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
  if (lane == 0) red_max[wid] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));

  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  float ls = 0.f;
  for (int i = wid; i < parts; i += 4) {
    const size_t r = slot(i) * g + h;
    const float wt = fast_exp2(p.ws_ml[r * 2] - M);
    ls = fmaf(wt, p.ws_ml[r * 2 + 1], ls);
    const float* a = p.ws_acc + r * D + lane * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = fmaf(wt, a[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) red_acc[wid][lane * EPT + e] = acc[e];
  if (lane == 0) red_l[wid] = ls;
  __syncthreads();
  if (wid == 0) {
    const float lsum = (red_l[0] + red_l[1]) + (red_l[2] + red_l[3]);
    float o[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = lane * EPT + e;
      o[e] = ((red_acc[0][i] + red_acc[1][i]) + (red_acc[2][i] + red_acc[3][i])) / lsum;
    }
    store_row<DT, EPT>((char*)p.out + ((size_t)s * p.num_heads + kv * g + h) * (D * EB) + lane * (EPT * EB), o);
  }
}

// The decode and merge kernels of one shape (nullptr if not compiled).
template <int DT, int D, int BS>
bool pick_group(int gp, const void** dec, const void** red) {
  *red = reinterpret_cast<const void*>(&reduce_kernel<DT, D>);
  switch (gp) {
    case 1: *dec = reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, 1>); return true;
    case 2: *dec = reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, 2>); return true;
    case 4: *dec = reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, 4>); return true;
    case 8: *dec = reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, 8>); return true;
    case 16: *dec = reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, 16>); return true;
    default: return false;
  }
}

template <int DT, int D>
bool pick_block(int bs, int gp, const void** dec, const void** red) {
  switch (bs) {
    case 8: return pick_group<DT, D, 8>(gp, dec, red);
    case 16: return pick_group<DT, D, 16>(gp, dec, red);
    case 32: return pick_group<DT, D, 32>(gp, dec, red);
    default: return false;
  }
}

template <int DT>
bool pick_decode_kernels(int head_dim, int bs, int gp, const void** dec, const void** red) {
  switch (head_dim) {
    case 64: return pick_block<DT, 64>(bs, gp, dec, red);
    case 128: return pick_block<DT, 128>(bs, gp, dec, red);
    default: return false;
  }
}

}  // namespace pagedkv
