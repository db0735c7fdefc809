// Launch parameters and kernel lookup of pa_decode (decode_kernel.h), shared by
// the decode kernels and their host code in decode_api.hip.  Internal.
#pragma once

#include "common.h"

namespace pagedkv {

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
};

// Decode kernel variants: K/V loads with the non-temporal hint (pa_decode), the same
// with the append of the newest tokens (pa_decode_append), and K/V loads with the
// default cache policy (pa_decode_cached).
enum class DecodeVariant { kStream, kAppend, kCached };

// The decode and merge kernels for one shape, one translation unit per element
// type; false for a shape outside the compiled set.  `gp` is the padded group.
bool decode_kernels_f32(int head_dim, int block_size, int gp, DecodeVariant variant,
                        const void** dec, const void** red);
bool decode_kernels_f16(int head_dim, int block_size, int gp, DecodeVariant variant,
                        const void** dec, const void** red);
bool decode_kernels_bf16(int head_dim, int block_size, int gp, DecodeVariant variant,
                         const void** dec, const void** red);

// Smallest group size of the compiled decode variants that can hold `group`
// query heads (1, 2, 4, 8, 16), or 0 if none can.
inline int padded_group(int group) {
  for (int g = 1; g <= 16; g *= 2)
    if (group <= g) return g;
  return 0;
}

}  // namespace pagedkv
