// Even split of one decode step's work over a fixed number of waves.
//
// The work of a decode step is cut into tiles of 16 consecutive tokens of one
// (sequence, KV head) pair.  Pair (s, kv) owns ceil(L_s / 16) tiles, and the
// tiles are numbered sequence by sequence, KV head by KV head, tile by tile:
//     pair (s, kv) starts at  Hkv * C_s + kv * n_s,   C_s = sum_{s' < s} n_s'.
// With T tiles in all and nw waves, wave w takes the tiles
//     [floor(w T / nw), floor((w + 1) T / nw)),
// so every wave reads the same number of K/V rows, give or take one tile,
// whatever the mix of lengths.  A wave's range is a run of "segments", each the
// part of one pair that falls inside it:
//   * a segment that covers its whole pair yields that pair's final output;
//   * otherwise the pair is split over several consecutive waves.  Each piece
//     yields a partial result (running max, running sum, unnormalised
//     accumulator): this is the same blockwise merge the softmax uses across
//     blocks, applied across waves, and a second kernel combines the pieces.
//     The wave that holds the pair's first tile "owns" the pair; its piece is
//     its last segment.  Every other piece is the first segment of its wave.
//
// Waves do not all run at the same speed (the oldest wave on a SIMD is issued
// first, and some XCDs are slower than others), so each share is cut into
// chunks: its head (all but the last 1/tail_div of it), which wave k processes
// first, and its tail, cut into `pieces` parts of halving size (1/2, 1/4, ...,
// the last one taking the rest).  Tail parts go to whichever wave asks first
// once its head is done, all shares' first parts before any second part, so the
// work handed out last is the smallest and the waves finish close together.
// With tail_div = 0 there are no tails.  Chunk c = k (pieces + 1) + r is the
// head (r = 0) or tail part r - 1 of share k, so chunks follow the tile order.
// Chunk boundaries are fixed by the lengths alone, so the result does not
// depend on which wave took which part.  Pieces and owners are defined per
// chunk exactly as above.
//
// Everything here is plain integer arithmetic shared by the kernels and by the
// host code that sizes the workspace.
#pragma once

#include <hip/hip_runtime.h>

namespace pagedkv {

constexpr int kTileTokens = 16;       // tokens per tile (the MFMA row count)
constexpr int kMinTilesPerWave = 8;   // fewer tiles per wave would only add partials
constexpr int kMaxWaves = 2048;       // 2 per SIMD of a 256-CU chip; the launch uses 1 per SIMD
constexpr int kMaxTailPieces = 4;     // tail parts per share, at most

__host__ __device__ inline int tiles_of(int len) { return (len + kTileTokens - 1) / kTileTokens; }

// Waves that get tiles when `launched` waves run over T tiles: at most one per
// kMinTilesPerWave tiles, so each has at least one tile (0 when T == 0).
__host__ __device__ inline long long waves_used(long long T, long long launched) {
  const long long want = (T + kMinTilesPerWave - 1) / kMinTilesPerWave;
  return want < launched ? want : launched;
}

// First tile of wave w (w = nw gives T).
__host__ __device__ inline long long wave_begin(long long w, long long T, long long nw) {
  return w * T / nw;
}

// The wave whose range holds tile t (0 <= t < T): the largest w with
// wave_begin(w) <= t, i.e. w T / nw < t + 1.
__host__ __device__ inline long long wave_of(long long t, long long T, long long nw) {
  return ((t + 1) * nw + T - 1) / T - 1;
}

// Tail parts shorter than this many tiles do not pay for the chunk start they cost,
// so the divisor of a call with short shares is lowered (to at least kMinTailDiv):
// with 1/16 of a 128-tile share a part would be 8 tiles.
constexpr int kMinTailTiles = 16;
constexpr int kMinTailDiv = 8;

// The tail divisor used for T tiles over nw shares when tail_div is asked for: at
// most tail_div, lowered toward kMinTailDiv while a part would have fewer than
// kMinTailTiles tiles (a function of T and nw only, so every kernel agrees).
__host__ __device__ inline int effective_tail_div(long long T, long long nw, int tail_div) {
  if (tail_div <= 0 || nw <= 0) return tail_div;
  long long d = T / nw / kMinTailTiles;
  if (d > tail_div) d = tail_div;
  const int floor_div = kMinTailDiv < tail_div ? kMinTailDiv : tail_div;
  return d < floor_div ? floor_div : (int)d;
}

// Chunk layout of one call: nw shares, each a head and `pieces` tail parts.
struct ChunkPlan {
  long long T;    // tiles of the step
  long long nw;   // shares (waves that get a head)
  int tail_div;   // 0 = no tails
  int pieces;     // tail parts per share, >= 1

  __host__ __device__ long long chunks() const { return nw * (pieces + 1); }

  // First tile of chunk c (c = chunks() gives T).
  __host__ __device__ long long begin(long long c) const {
    const long long k = c / (pieces + 1);
    const int r = (int)(c - k * (pieces + 1));
    const long long b = wave_begin(k, T, nw);
    if (r == 0) return b;
    const long long e = wave_begin(k + 1, T, nw);
    const long long tail = tail_div > 0 ? (e - b) / tail_div : 0;
    return e - tail + (tail - (tail >> (r - 1)));  // part r-1 starts after 1 - 2^-(r-1) of the tail
  }

  // The chunk holding tile t (0 <= t < T): the largest c with begin(c) <= t, so
  // an empty chunk is never returned.
  __host__ __device__ long long chunk_of(long long t) const {
    const long long k = wave_of(t, T, nw);
    const long long c0 = k * (pieces + 1);
    for (int r = pieces; r > 0; --r)
      if (begin(c0 + r) <= t) return c0 + r;
    return c0;
  }

  // Chunk of tail ticket t (0 <= t < pieces * nw): the first parts of all shares,
  // then the second parts, and so on.
  __host__ __device__ long long ticket_chunk(long long t) const {
    const long long part = t / nw;
    const long long k = t - part * nw;
    return k * (pieces + 1) + 1 + part;
  }
};

// Position of one tile in pair order: sequence s (length L, n tiles), KV head
// kv, tile j of the pair.
struct TileCursor {
  int s, kv, j, n, L;

  // Step to the next tile of the batch (the next tile of the pair, else the
  // first tile of the next KV head, else of the next non-empty sequence).
  // Returns false, leaving n = 0, when there is none; num_seqs bounds every read.
  template <class LenFn>
  __host__ __device__ bool next(int num_seqs, int num_kv_heads, LenFn len) {
    if (++j < n) return true;
    j = 0;
    if (++kv < num_kv_heads) return true;
    kv = 0;
    do {
      if (++s >= num_seqs) {
        n = 0;
        return false;
      }
      L = len(s);
    } while (L == 0);
    n = tiles_of(L);
    return true;
  }
};

// Walk the tiles [t0, t1) of one chunk, starting in pair (s, kv) at tile j of
// that pair.  len(s) gives the length of sequence s (already clamped); seg(s,
// kv, jb, je, L) is called for each segment, tiles [jb, je) of pair (s, kv).
// The caller guarantees that tile t0 is tile j of pair (s, kv) and t1 <= T,
// so the walk never runs past the last non-empty sequence; it still stops at
// num_seqs rather than read past the lengths.
template <class LenFn, class SegFn>
__host__ __device__ inline void walk_tiles(long long t0, long long t1, int s, int kv, int j,
                                           int num_seqs, int num_kv_heads, LenFn len, SegFn seg) {
  int L = len(s);
  int n = tiles_of(L);
  long long t = t0;
  while (t < t1) {
    const long long left = t1 - t;
    const int je = left < (long long)(n - j) ? j + (int)left : n;
    if (je <= j) return;  // cannot happen for a valid start; never loop without progress
    seg(s, kv, j, je, L);
    t += je - j;
    if (t >= t1) break;
    // je == n here: the pair is done, go to the next one
    j = 0;
    if (++kv == num_kv_heads) {
      kv = 0;
      do {
        if (++s >= num_seqs) return;
        L = len(s);
      } while (L == 0);
      n = tiles_of(L);
    }
  }
}

}  // namespace pagedkv
