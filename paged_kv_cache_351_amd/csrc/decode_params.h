// Launch parameters and kernel lookup of pa_decode (decode_kernel.h), shared by
// the decode kernels and their host code in decode_api.hip.  Internal.
#pragma once

#include "common.h"
#include "pagedkv.h"

namespace pagedkv {

// Batches of at most this many sequences keep every sequence's length and tile
// prefix sum in LDS (each wave its own copy), so locating a chunk and stepping to
// the next sequence read LDS instead of global memory.
constexpr int kLdsSeqs = 2048;

// Everything one pa_decode launch needs, already validated by the host code.
struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  int* ws_meta;        // 64-int header, then [chunks][4]: per chunk, the pair it
                       // owns, how many chunks share it, whether it left a first piece
  float* ws_ml;        // [2 * chunks][group][2]: running max and sum of each piece
  float* ws_acc;       // [2 * chunks][group][head_dim]: unnormalised accumulator
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;           // num_heads / num_kv_heads
  int head_dim;
  int block_size;
  int num_blocks;
  int max_blocks_per_seq;
  int max_seq_len;
  int num_waves;       // decode waves launched
  int tail_div;        // the last 1/tail_div of each wave's share is handed out on
                       // demand; 0 = none
  int tail_pieces;     // parts the tail is cut into (halving sizes), 1..kMaxTailPieces
  float scale_log2e;   // scale * log2(e): logits are taken in base 2
  // pa_decode_append only (null otherwise): the K and V rows of each sequence's newest
  // token, position seq_lens[s] - 1, as [num_seqs][num_kv_heads][head_dim].  The decode
  // kernel reads that token from here; the merge kernel's last append_blocks
  // workgroups then store these rows into their slots of the caches.
  const void* new_k;
  const void* new_v;
  int merge_blocks;    // workgroups of the merge kernel that merge (one wave per chunk)
  int append_blocks;   // workgroups after them that store the newest rows (0 = none)
  // pa_multi_query on the decode kernels (null otherwise): query rows of sequence s are
  // q_start[s] .. q_start[s+1] - 1 of q and out, and row r of pair (s, kv) is query
  // r / group, head r % group, seeing the tokens up to its own position.
  const int32_t* q_start;
  int rows;            // rows of one (sequence, KV head) pair: group, or the multi-query
                       // rows (max_q_len * group, at most 16)
  int total_q;         // rows mode: query rows of q and out (q_start values are clamped
                       // to [0, total_q], so no access leaves them)
  // Rows mode over shared-prefix groups (0 otherwise): a "sequence" is a block of one
  // group's members and its block table is the group's laid-out table (shared_rows): the
  // prefix once, then each member's own tokens, each region starting on a tile.  Every
  // entry is a block id (bits 0..21) with the owner of its tokens (bits 27..31: the
  // member's row index, kSharedAll for the prefix) and, less one, how many of the
  // region's tokens lie at or after the block's start, at most 32 (bits 22..26).  Row r
  // sees the prefix and its own region only.
  int shared;
};

// Bits of a laid-out shared-prefix table entry.
constexpr int kSharedIdBits = 22;
constexpr unsigned kSharedIdMask = (1u << kSharedIdBits) - 1u;
constexpr int kSharedEndShift = 22;     // 5 bits: tokens of the region from the block start, - 1
constexpr int kSharedOwnerShift = 27;   // 5 bits: member row index 0..15, or kSharedAll
constexpr int kSharedAll = 16;   // owner of the prefix blocks: every row

// Decode kernel variants: K/V loads with the non-temporal hint (pa_decode), the same
// with the append of the newest tokens (pa_decode_append), and K/V loads with the
// default cache policy (pa_decode_cached).
enum class DecodeVariant { kStream, kAppend, kCached, kRows };

// The decode and merge kernels for one shape, one translation unit per element
// type; false for a shape outside the compiled set.  `gp` is the padded group.
bool decode_kernels_f32(int head_dim, int block_size, int gp, DecodeVariant variant,
                        const void** dec, const void** red);
bool decode_kernels_f16(int head_dim, int block_size, int gp, DecodeVariant variant,
                        const void** dec, const void** red);
bool decode_kernels_bf16(int head_dim, int block_size, int gp, DecodeVariant variant,
                         const void** dec, const void** red);

// pa_multi_query on the decode kernels ("rows mode"): when every (sequence, KV head)
// pair has at most 16 (query, head) rows, the batch's tables fit the decode kernel's
// LDS (at most kLdsSeqs sequences, tile prefix sums below 2^31) and the decode kernels
// cover the shape, each
// pair's rows take the 16 columns of the decode kernel's score tile, every row with its
// own causal limit, and the work is split evenly over the waves as for pa_decode.
// `multi_query_rows_apply` says whether the mode covers the shape; the workspace it
// needs is `multi_query_rows_workspace` bytes (any 16-byte aligned buffer: the call
// clears the part it counts on).  Launches a header clear, the decode kernel and the
// merge kernel on `st`.
bool multi_query_rows_apply(pa_dtype dtype, int num_seqs, int num_heads, int num_kv_heads,
                            int head_dim, int block_size, int max_q_len, int max_seq_len);
size_t multi_query_rows_workspace(int num_seqs, int num_kv_heads, int head_dim, int max_seq_len,
                                  int rows);
pa_status multi_query_rows(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* q_start, int num_seqs, int total_q, int num_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_q_len, int max_seq_len, float scale,
                           pa_dtype dtype, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t st);

// pa_decode_shared_prefix on the decode kernels: each group's members are taken in
// blocks of at most 16 / group; for every block a layout kernel writes one table whose
// first entries are the group's prefix blocks (once) followed by each member's own
// blocks, every member's region starting on a whole tile (16 tokens, or a 32-token
// block), and the rows mode runs over those tables with the members as its rows.
// `shared_rows_apply` says whether the path covers the call; it needs
// `shared_rows_workspace` bytes (16-byte aligned, no zero-fill) for the given block size.
bool shared_rows_apply(pa_dtype dtype, int num_groups, int num_heads, int num_kv_heads,
                       int head_dim, int block_size, int num_blocks, int max_group_size,
                       int max_seq_len);
size_t shared_rows_workspace(int num_seqs, int num_groups, int num_heads, int num_kv_heads,
                             int head_dim, int block_size, int max_group_size, int max_seq_len);
pa_status shared_rows(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* seq_lens,
                      const int32_t* group_start, const int32_t* prefix_lens, int num_seqs,
                      int num_groups, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int max_blocks_per_seq, int max_group_size,
                      int max_seq_len, float scale, pa_dtype dtype, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t st);

// Smallest group size of the compiled decode variants that can hold `group`
// query heads (1, 2, 4, 8, 16), or 0 if none can.
inline int padded_group(int group) {
  for (int g = 1; g <= 16; g *= 2)
    if (group <= g) return g;
  return 0;
}

}  // namespace pagedkv
