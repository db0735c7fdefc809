// Host check of the even tile split used by the decode kernel (split.h).
//
// For seeded random batches (empty sequences, partial tiles, long sequences, more
// waves than tiles, with and without tails cut into 1-4 parts) it replays what the
// kernel does for every chunk (the head and the tail parts of each wave's share)
// -- locate its first tile, walk its segments -- and checks that:
//   * tail tickets name every tail part once, all first parts before any second;
//   * every tile of every (sequence, KV head) pair is visited exactly once, and
//     the chunks' ranges cover [0, T) in order (tail chunks may be empty);
//   * a segment never leaves its pair, and segments follow the pair order;
//   * the tile-by-tile cursor the kernel uses visits the same tiles in order;
//   * a split pair has exactly one owner (the piece holding its first tile), which
//     is its chunk's last segment; every other piece is its chunk's first segment;
//   * the pieces the merge step reads for an owned pair (slot 2c+1 of the owner
//     chunk c, then slot 2c' of every chunk c' = c+1 .. c+parts-1 that wrote a
//     first piece) are exactly that pair's pieces and together cover its tiles.
// Prints "split ok: <cases>" and exits 0, or prints the first failure and exits 1.
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "split.h"

using namespace pagedkv;

struct Piece {
  int s, kv, jb, je;
};

static int fail(const char* what, int c) {
  printf("split check failed (case %d): %s\n", c, what);
  return 1;
}

// td < 0: the kernels' default, effective_tail_div(T, nw, -td)
int check(const std::vector<int>& lens, int Hkv, long long launched, int c, int td, int pieces) {
  const int N = (int)lens.size();
  std::vector<long long> C(N + 1, 0);  // C[s] = tiles of sequences before s
  for (int s = 0; s < N; ++s) C[s + 1] = C[s] + tiles_of(lens[s]);
  const long long T = C[N] * Hkv;
  const long long nw = waves_used(T, launched);
  if (T > 0 && (nw < 1 || nw > launched || nw > T)) return fail("waves_used out of range", c);
  if (T == 0 && nw != 0) return fail("waves for an empty batch", c);

  std::vector<int> seen(T, 0);  // visits of each tile, by its global index
  if (td < 0) {
    const int want = -td;
    td = effective_tail_div(T, nw, want);
    if (T > 0 && (td > want || td < (want < kMinTailDiv ? want : kMinTailDiv)))
      return fail("effective tail divisor out of range", c);
  }
  const ChunkPlan plan{T, nw, td, pieces};
  const long long nc = plan.chunks();
  // tail tickets name every tail chunk exactly once, first parts first
  {
    std::vector<int> got(nc, 0);
    long long prev_part = -1;
    for (long long t = 0; t < (long long)pieces * nw; ++t) {
      const long long ch = plan.ticket_chunk(t);
      if (ch < 0 || ch >= nc || ch % (pieces + 1) == 0) return fail("ticket names a head or no chunk", c);
      const long long part = ch % (pieces + 1) - 1;
      if (part < prev_part) return fail("tickets not in part order", c);
      prev_part = part;
      got[ch]++;
    }
    for (long long ch = 0; ch < nc; ++ch)
      if ((ch % (pieces + 1) == 0) == (got[ch] == 1)) return fail("tickets do not cover the tails once", c);
  }
  std::vector<Piece> first(nc, Piece{-1, -1, -1, -1}), owned(nc, Piece{-1, -1, -1, -1});
  std::vector<int> parts(nc, 0);
  long long covered = 0;
  for (long long w = 0; w < nc; ++w) {
    const long long t0 = plan.begin(w), t1 = plan.begin(w + 1);
    if (t0 != covered || t1 < t0) return fail("chunk ranges do not tile [0, T)", c);
    const bool head = w % (pieces + 1) == 0;
    if (t1 == t0 && head) return fail("empty head chunk", c);
    if (td == 0 && !head && t1 != t0) return fail("tail chunk without tails", c);
    if (t1 == t0) continue;
    if (plan.chunk_of(t0) != w || plan.chunk_of(t1 - 1) != w) return fail("chunk_of mismatch", c);
    // locate tile t0 as the kernel does: the first sequence whose tiles end past t0
    int s0 = 0;
    while (C[s0 + 1] * Hkv <= t0) ++s0;
    const long long off = t0 - C[s0] * Hkv;
    const int n0 = tiles_of(lens[s0]);
    int nseg = 0, last_jb = -1, last_je = -1, last_s = -1, last_kv = -1;
    long long t_seg = t0;
    bool bad = false;
    const char* why = "";
    walk_tiles(t0, t1, s0, (int)(off / n0), (int)(off % n0), N, Hkv,
               [&](int s) { return lens[s]; },
               [&](int s, int kv, int jb, int je, int L) {
                 const int n = tiles_of(L);
                 if (L != lens[s] || jb < 0 || je > n || jb >= je) { bad = true; why = "segment bounds"; }
                 if (C[s] * Hkv + (long long)kv * n + jb != t_seg) { bad = true; why = "segment position"; }
                 for (int j = jb; j < je; ++j) seen[C[s] * Hkv + (long long)kv * n + j]++;
                 if (jb > 0 && nseg != 0) { bad = true; why = "non-owned piece is not the first segment"; }
                 if (nseg == 0 && jb > 0) first[w] = Piece{s, kv, jb, je};
                 if (nseg == 0 && jb == 0 && je < n) first[w] = Piece{-1, -1, -1, -1};
                 if (jb == 0 && je < n) {
                   owned[w] = Piece{s, kv, jb, je};
                   parts[w] = (int)(plan.chunk_of(t_seg + n - 1) - w + 1);
                 }
                 last_jb = jb;
                 last_je = je;
                 last_s = s;
                 last_kv = kv;
                 t_seg += je - jb;
                 ++nseg;
               });
    if (bad) return fail(why, c);
    if (t_seg != t1) return fail("walk does not end at the range end", c);
    // the tile-by-tile cursor (the kernel's load and compute order) visits the
    // same tiles in the same order as the segment walk
    {
      TileCursor cur{s0, (int)(off / n0), (int)(off % n0), n0, lens[s0]};
      for (long long t = t0; t < t1; ++t) {
        if (C[cur.s] * Hkv + (long long)cur.kv * cur.n + cur.j != t || cur.n != tiles_of(lens[cur.s]))
          return fail("cursor position", c);
        const bool more = cur.next(N, Hkv, [&](int s) { return lens[s]; });
        if (t + 1 < T && !more) return fail("cursor ended early", c);
        if (t + 1 == T && more) return fail("cursor ran past the last tile", c);
      }
    }
    if (owned[w].s >= 0 && (owned[w].s != last_s || owned[w].kv != last_kv || last_jb != 0 ||
                            last_je != owned[w].je))
      return fail("owned piece is not the last segment", c);
    if (owned[w].s >= 0 && parts[w] < 2) return fail("owned split pair with fewer than 2 pieces", c);
    covered = t1;
  }
  if (covered != T) return fail("ranges stop before T", c);
  // every tile exactly once (the position check above maps each visit to its
  // pair's own index range, so a count of one everywhere means exact coverage)
  for (long long t = 0; t < T; ++t)
    if (seen[t] != 1) return fail("tile not visited exactly once", c);
  // the merge step's reads: chunks that wrote no first piece (empty tails) are skipped
  int owners = 0;
  for (long long w = 0; w < nc; ++w) {
    if (owned[w].s < 0) continue;
    ++owners;
    const Piece o = owned[w];
    const int n = tiles_of(lens[o.s]);
    int next = o.je;
    for (int i = 1; i < parts[w]; ++i) {
      const long long v = w + i;
      if (v >= nc) return fail("merge reads past the last chunk", c);
      const Piece f = first[v];
      if (f.s < 0) {
        if (plan.begin(v) != plan.begin(v + 1))
          return fail("merge skips a non-empty chunk", c);
        continue;
      }
      if (f.s != o.s || f.kv != o.kv || f.jb != next) return fail("merge piece mismatch", c);
      next = f.je;
    }
    if (next != n) return fail("merge pieces do not cover the pair", c);
  }
  // every split pair has an owner: count pairs whose tiles span more than one wave
  int split_pairs = 0;
  for (int s = 0; s < N; ++s)
    for (int kv = 0; kv < Hkv; ++kv) {
      const int n = tiles_of(lens[s]);
      if (n == 0) continue;
      const long long a = C[s] * Hkv + (long long)kv * n;
      if (plan.chunk_of(a) != plan.chunk_of(a + n - 1)) ++split_pairs;
    }
  if (split_pairs != owners) return fail("split pairs and owners differ", c);
  return 0;
}

int main() {
  std::mt19937 rng(12345);
  int cases = 0;
  const long long launched_set[] = {1, 2, 3, 7, 64, 1000, 3072, 8192};
  const int hkv_set[] = {1, 2, 3, 8};
  for (int rep = 0; rep < 200; ++rep) {
    const int kind = rep % 4;
    const int N = 1 + (int)(rng() % (rep < 100 ? 12 : (kind == 3 ? 40 : 300)));
    std::vector<int> lens(N);
    for (int& L : lens) {
      const unsigned r = rng();
      if (kind == 0) L = (int)(r % 40);                       // short, many empty and partial
      else if (kind == 1) L = (r % 5 == 0) ? 0 : (int)(r % 4097);
      else if (kind == 2) L = 512 + (int)(r % 3585);          // the Llama-3-8B mix
      else L = (r % 3 == 0) ? (int)(r % 17) : 8192 + (int)(r % 24577);
    }
    for (int Hkv : hkv_set)
      for (long long launched : launched_set)
        for (int td : {0, 4, 8, -16})
          for (int pieces : {1, 3, 4}) {
            if (td == 0 && pieces != 1) continue;
            if (check(lens, Hkv, launched, cases, td, pieces)) return 1;
            ++cases;
          }
  }
  // all empty, single token, one huge sequence
  for (int td : {0, 8, -16})
    for (int pieces : {1, 3}) {
      if (check(std::vector<int>(5, 0), 2, 3072, cases++, td, pieces)) return 1;
      if (check(std::vector<int>{1}, 1, 3072, cases++, td, pieces)) return 1;
      if (check(std::vector<int>{0, 0, 1, 0}, 8, 3072, cases++, td, pieces)) return 1;
      if (check(std::vector<int>{32768}, 8, 3072, cases++, td, pieces)) return 1;
    }
  printf("split ok: %d cases\n", cases);
  return 0;
}
