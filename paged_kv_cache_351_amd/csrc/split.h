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
// first, and some XCDs are slower than others), so each share can be cut into
// two chunks: its head (all but the last 1/tail_div of it), which wave k
// processes first, and its tail, which goes to whichever wave asks first once
// its own head is done (tail_div = 0: no tails, every share is one chunk).
// Chunk 2k is the head of share k and chunk 2k+1 its tail; chunk boundaries are
// fixed by the lengths alone, so the result does not depend on which wave took
// which tail.  Pieces and owners are defined per chunk exactly as above.
//
// Everything here is plain integer arithmetic shared by the kernels and by the
// host code that sizes the workspace.
#pragma once

#include <hip/hip_runtime.h>

namespace pagedkv {

constexpr int kTileTokens = 16;       // tokens per tile (the MFMA row count)
constexpr int kMinTilesPerWave = 8;   // fewer tiles per wave would only add partials
constexpr int kMaxWaves = 4096;       // 4 per SIMD of a 256-CU chip; the launch uses 1 per SIMD

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

// First tile of chunk c (c = 2 nw gives T).  Chunk 2k is the head of share k,
// chunk 2k+1 its last (length / tail_div) tiles, which may be none.
__host__ __device__ inline long long chunk_begin(long long c, long long T, long long nw, int tail_div) {
  const long long k = c >> 1;
  const long long b = wave_begin(k, T, nw);
  if ((c & 1) == 0) return b;
  const long long e = wave_begin(k + 1, T, nw);
  return tail_div > 0 ? e - (e - b) / tail_div : e;
}

// The chunk holding tile t (0 <= t < T): the largest c with chunk_begin(c) <= t,
// so an empty chunk is never returned.
__host__ __device__ inline long long chunk_of(long long t, long long T, long long nw, int tail_div) {
  const long long k = wave_of(t, T, nw);
  return 2 * k + (t >= chunk_begin(2 * k + 1, T, nw, tail_div) ? 1 : 0);
}

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
