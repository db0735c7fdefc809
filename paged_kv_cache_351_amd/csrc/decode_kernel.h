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
// Work decomposition
//   One 64-lane wave (= one workgroup) per (KV head, sequence, context
//   partition).  A partition is part_tokens consecutive tokens (a multiple of the
//   block size); the wave walks it in tiles of 16 tokens.  Every query head of
//   the KV head's group (g = num_heads / num_kv_heads <= GP) is handled by the
//   same wave, so each K/V row is read from HBM once.
//   Grid order: x = KV head, y = sequence, z = partition.  Workgroups are handed
//   to the eight XCDs round-robin in linear order, so consecutive ids must carry
//   similar work: with the partition index slowest, every XCD gets a fair share
//   of first partitions (which every sequence has) and of late ones (which only
//   long sequences have), and the empty tail partitions come last.  With the
//   partition index fastest instead, partition p would always land on XCD p mod 8
//   and the chip would run at the speed of its busiest XCD.
//
// Lane roles (lane = 16 * grp + col, grp = 0..3, col = 0..15)
//   q.K^T on the matrix cores: v_mfma_f32_16x16x32_{bf16,f16} (or 16x16x4_f32)
//     with A = the tile's K rows (row = token col, this lane's 16-byte chunks
//     4c + grp of the row) and B = the group's query rows padded to 16 columns
//     (column = head col, same chunks).  Any fixed assignment of head_dim
//     positions to MFMA k-slots gives the same dot products, so the chunking
//     only has to match between A and B.  The result lands as
//     S[token 4*grp + r][head col], r = 0..3, in lane (grp, col).
//   Online softmax: lane (grp, col) keeps its own running max m and sum l for
//     head col over the tokens 4*grp + r of every tile, i.e. four independent
//     streams per head; they are merged once at the end of the partition.
//   P.V on the vector ALU: lane (grp, col) owns head_dim/16 consecutive
//     elements (at col * head_dim/16) of tokens 4*grp + j, j = 0..3, and
//     accumulates acc[h][.] for every head h of the group.  The weight p of
//     (head h, token 4*grp + j) sits in lane (grp, h); DPP row_newbcast:h
//     broadcasts it to the 16 lanes of the row -- no LDS, no barrier.
//
// Partition result
//   A sequence with a single partition writes its normalised output directly.
//   Otherwise each partition stores (m, l) and the unnormalised acc in float32
//   and reduce_kernel merges them in a fixed order (deterministic).
//
// Logits are taken in base 2 (scale * log2 e folded in), so every exponential is
// one v_exp_f32.  Running maxima start at a finite -1e30 so that a stream with
// no valid token yet never forms inf - inf.  Tokens past the sequence end in the
// last tile are redirected to the sequence's last token before loading (so no
// unused slot is ever read) and their scores are replaced by -inf with a select,
// which makes their weights exactly 0.
#pragma once

#include <type_traits>

#include "common.h"

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
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      u32x4 w = {__float_as_uint(v[i]), __float_as_uint(v[i + 1]), __float_as_uint(v[i + 2]),
                 __float_as_uint(v[i + 3])};
      reinterpret_cast<u32x4*>(dst)[i / 4] = w;
    }
  } else {
    uint32_t w[N / 2];
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
    if constexpr (N / 2 == 4) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    } else if constexpr (N / 2 == 2) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
    } else {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) reinterpret_cast<uint32_t*>(dst)[i] = w[i];
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
  const int kvh = blockIdx.x;
  const int s = blockIdx.y;
  const int part = blockIdx.z;
  const int g = p.group;
  const int head0 = kvh * g;
  const int P = p.part_tokens;

  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int nparts = (L + P - 1) / P;

  if (L == 0) {  // nothing to attend to: zeros
    if (part == 0) {
      char* o = (char*)p.out + ((size_t)s * p.num_heads + head0) * ROWB;
      for (int i = lane; i < g * D; i += 64) {
        if constexpr (DT == kF32) reinterpret_cast<float*>(o)[i] = 0.f;
        else reinterpret_cast<uint16_t*>(o)[i] = 0;
      }
    }
    return;
  }
  if (part >= nparts) return;

  const int tok0 = part * P;
  const int n_tok = min(P, L - tok0);

  // Physical ids of this partition's blocks, one per lane (<= 64 by construction).
  // An id outside the pool is a contract violation; it is replaced by 0 so that
  // no access can leave the pool.
  int my_id = 0;
  {
    const int nblk = (n_tok + BS - 1) / BS;
    if (lane < nblk) {
      const int id = p.block_tables[(size_t)s * p.max_blocks_per_seq + tok0 / BS + lane];
      my_id = (unsigned)id < (unsigned)p.num_blocks ? id : 0;
    }
  }

  const size_t tok_stride = (size_t)p.num_kv_heads * ROWB;
  const size_t blk_bytes = (size_t)BS * tok_stride;
  const char* kbase = (const char*)p.k_cache + (size_t)kvh * ROWB;
  const char* vbase = (const char*)p.v_cache + (size_t)kvh * ROWB + col * (VE * EB);

  // Query fragments (MFMA B operand): head head0 + col, chunks 4c + grp.
  u32x4 qf[NKC];
  {
    const char* qrow = (const char*)p.q + ((size_t)s * p.num_heads + head0 + col) * ROWB;
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      qf[c] = col < g ? *reinterpret_cast<const u32x4*>(qrow + (4 * c + grp) * 16) : u32x4{0, 0, 0, 0};
  }

  struct Tile {
    u32x4 k[NKC];
    uint32_t v[4][VW];
  };

  // Tile tt covers partition tokens [16 tt, 16 tt + 16).  A token index past the
  // partition's last token is clamped to that token, so every load reads a real
  // row of this sequence (never an unused slot); such tokens get weight exactly 0
  // from the score mask below.  Loads are therefore always legal, and the
  // prefetch of a tile past the end simply re-reads the last one (cache hits).
  const int last = n_tok - 1;
  auto load_tile = [&](Tile& T, int tt) __attribute__((always_inline)) {
    const int t0 = 16 * tt;
    const int tk = min(t0 + col, last);        // K row of this lane
    int tv[4];                                 // V rows of this lane
#pragma unroll
    for (int j = 0; j < 4; ++j) tv[j] = min(t0 + 4 * grp + j, last);
    int pk, pv[4];
    if constexpr (BS == 8) {
      const int ida = __builtin_amdgcn_readlane(my_id, 2 * tt);
      const int idb = __builtin_amdgcn_readlane(my_id, 2 * tt + 1);
      pk = (tk & 8) ? idb : ida;
#pragma unroll
      for (int j = 0; j < 4; ++j) pv[j] = (tv[j] & 8) ? idb : ida;
    } else {
      const int id = __builtin_amdgcn_readlane(my_id, t0 / BS);
      pk = id;
#pragma unroll
      for (int j = 0; j < 4; ++j) pv[j] = id;
    }
    const char* kp = kbase + (size_t)pk * blk_bytes + (size_t)(tk % BS) * tok_stride;
#pragma unroll
    for (int c = 0; c < NKC; ++c) T.k[c] = *reinterpret_cast<const u32x4*>(kp + (4 * c + grp) * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      load_dwords<VW>(vbase + (size_t)pv[j] * blk_bytes + (size_t)(tv[j] % BS) * tok_stride, T.v[j]);
  };

  float m = kNegBig;
  float l = 0.f;
  float acc[GP][VE];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[h][e] = 0.f;
  const float sl2 = p.scale_log2e;

  auto compute = [&](const Tile& T, int tt) __attribute__((always_inline)) {
    // S = K q^T on the matrix cores
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      if constexpr (DT == kBF16) {
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T.k[c]),
                                                     __builtin_bit_cast(bf16x8, qf[c]), sc, 0, 0, 0);
      } else if constexpr (DT == kF16) {
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, T.k[c]),
                                                    __builtin_bit_cast(f16x8, qf[c]), sc, 0, 0, 0);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(T.k[c][e]), __uint_as_float(qf[c][e]),
                                                    sc, 0, 0, 0);
      }
    }
    // online softmax, stream (grp, head col); tokens past the end get -inf
    const int lim = n_tok - 16 * tt - 4 * grp;
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
      unpack<DT, VW>(T.v[j], vf);
      static_for<GP>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const float pj = row_bcast<h>(pr[j]);
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[h][e] = fmaf(pj, vf[e], acc[h][e]);
      });
    }
  };

  // Two tiles in flight: while one is reduced the next two are being fetched.  The
  // loads are unconditional (clamped tile index) so no tile register is ever
  // copied, and the scheduling barriers keep a refill after the last use of the
  // registers it overwrites.
  const int n_tiles = (n_tok + 15) >> 4;
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
      float a = acc[h][e] * fh;
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[h][e] = a;
    }
  });

  if (nparts == 1) {
    // every row now holds the full sums; row grp stores heads h = grp (mod 4)
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
    const size_t row0 = (size_t)s * p.num_heads + head0;
    static_for<GP>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      if (h < g && (h & 3) == grp) {
        float* dst = p.ws_acc + ((row0 + h) * p.max_parts + part) * D + col * VE;
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          *reinterpret_cast<f32x4*>(dst + e) = f32x4{acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]};
      }
    });
    if (grp == 0 && col < g) {
      float* ml = p.ws_ml + ((row0 + col) * p.max_parts + part) * 2;
      ml[0] = M;
      ml[1] = ls;
    }
  }
}

// Merge the partition results of every (sequence, head) with more than one
// partition: M = max_p m_p, w_p = 2^(m_p - M), out = sum_p w_p acc_p / sum_p w_p l_p,
// summed in partition order.
template <int DT, int D>
__global__ __launch_bounds__(64) void reduce_kernel(DecodeParams p) {
  constexpr int EPT = D / 64;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int t = threadIdx.x;
  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int np = (L + p.part_tokens - 1) / p.part_tokens;
  if (np <= 1) return;
  const size_t row = (size_t)s * p.num_heads + h;
  const float* ml = p.ws_ml + row * p.max_parts * 2;
  float M = kNegBig;
  for (int i = 0; i < np; ++i) M = fmaxf(M, ml[2 * i]);
  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  float ls = 0.f;
  for (int i = 0; i < np; ++i) {
    const float w = fast_exp2(ml[2 * i] - M);
    ls = fmaf(w, ml[2 * i + 1], ls);
    const float* a = p.ws_acc + (row * p.max_parts + i) * D + t * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = fmaf(w, a[e], acc[e]);
  }
  constexpr int EB = Elem<DT>::bytes;
  char* o = (char*)p.out + row * (D * EB) + t * (EPT * EB);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const float v = acc[e] / ls;
    if constexpr (DT == kF32) reinterpret_cast<float*>(o)[e] = v;
    else if constexpr (DT == kBF16) reinterpret_cast<__bf16*>(o)[e] = (__bf16)v;
    else reinterpret_cast<_Float16*>(o)[e] = (_Float16)v;
  }
}

template <int DT, int D, int BS, int GP>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  DecodeParams args = p;
  void* kargs[] = {&args};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_kernel<DT, D, BS, GP>),
                                 dim3(p.num_kv_heads, p.num_seqs, p.max_parts), dim3(64), kargs, 0, stream);
  if (e != hipSuccess || p.max_parts == 1) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&reduce_kernel<DT, D>),
                         dim3(p.num_heads, p.num_seqs), dim3(64), kargs, 0, stream);
}

template <int DT, int D, int BS>
hipError_t dispatch_group(const DecodeParams& p, hipStream_t stream) {
  switch (padded_group(p.group)) {
    case 1: return launch_one<DT, D, BS, 1>(p, stream);
    case 2: return launch_one<DT, D, BS, 2>(p, stream);
    case 4: return launch_one<DT, D, BS, 4>(p, stream);
    case 8: return launch_one<DT, D, BS, 8>(p, stream);
    case 16: return launch_one<DT, D, BS, 16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t dispatch_block(const DecodeParams& p, hipStream_t stream) {
  switch (p.block_size) {
    case 8: return dispatch_group<DT, D, 8>(p, stream);
    case 16: return dispatch_group<DT, D, 16>(p, stream);
    case 32: return dispatch_group<DT, D, 32>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t dispatch_decode(const DecodeParams& p, hipStream_t stream) {
  switch (p.head_dim) {
    case 64: return dispatch_block<DT, 64>(p, stream);
    case 128: return dispatch_block<DT, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pagedkv
