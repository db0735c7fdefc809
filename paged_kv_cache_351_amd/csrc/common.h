// Internal declarations shared by the HIP kernels and the C-ABI host code of
// libpagedkv.  Not part of the public interface (that is include/pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pagedkv {

enum ElemType { kF32 = 0, kF16 = 1, kBF16 = 2 };

inline int elem_bytes(int dt) { return dt == kF32 ? 4 : 2; }

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
};

// The decode and merge kernels for one shape, one translation unit per element
// type; false for a shape outside the compiled set.  `gp` is the padded group.
bool decode_kernels_f32(int head_dim, int block_size, int gp, const void** dec, const void** red);
bool decode_kernels_f16(int head_dim, int block_size, int gp, const void** dec, const void** red);
bool decode_kernels_bf16(int head_dim, int block_size, int gp, const void** dec, const void** red);

hipError_t launch_write_kv(const void* k, const void* v, const int32_t* slots,
                           void* k_cache, void* v_cache, int num_tokens,
                           int row_bytes, long long pool_slots, hipStream_t stream);

hipError_t launch_copy_blocks(const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                              const int32_t* pairs, int num_pairs, long long block_bytes,
                              int src_blocks, int dst_blocks, hipStream_t stream);

// Everything one pa_multi_query launch needs, already validated by the host code.
struct MultiQueryParams {
  const void* q;               // [total_q][num_heads][head_dim]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;     // tokens in the cache, including the queries' own
  const int32_t* q_start;      // [num_seqs + 1] query row offsets; shared-prefix decode:
                               // [num_groups + 1] first member sequence of each group
  const int32_t* prefix_lens;  // shared-prefix decode: [num_groups] shared tokens
  void* out;                   // [total_q][num_heads][head_dim]
  const int32_t* order;        // [num_seqs]: items' sequences (groups), longest first, or
                               // null: workgroups in XCD-major order instead
  int32_t* order_out;          // where the ordering pass writes `order`
  float* ws_ml;                // [total_q * num_heads][parts][2] running max and sum
  float* ws_acc;               // [total_q * num_heads][parts][head_dim]
  int num_seqs;
  int total_q;
  int num_heads;
  int num_kv_heads;
  int group;
  int head_dim;
  int block_size;
  float inv_block_size;        // 1 / block_size, rounded to nearest
  int num_blocks;
  int max_blocks_per_seq;
  int max_q_len;
  int max_seq_len;
  int tq;                      // query tokens (or group members) per workgroup:
                               // its rows (16, 64 or 128) / group
  int qblocks;                 // query blocks per (sequence, KV head): ceil(max_q_len / tq)
  int parts;                   // context partitions; 1 = no merge step
  long long items;             // num_seqs * num_kv_heads * qblocks
  float scale_log2e;
};

// The pass that orders the items' sequences (shared: groups) longest first.
const void* multi_query_order_kernel(bool shared);

// The multi-query and partition-merge kernels for one element type and head_dim.
// rows = query rows per workgroup: 16 (the four waves split the context; 16-bit
// types), 64 or 128 (16 or 32 rows per wave sharing K/V tiles); `shared` picks the
// shared-prefix decode (16 rows, 16-bit types).
bool multi_query_kernels(int dtype, int head_dim, int rows, bool shared, const void** main,
                         const void** merge);

// Message returned by pa_last_error() on the calling thread.
void set_last_error(const char* msg);

// Smallest group size of the compiled decode variants that can hold `group`
// query heads (1, 2, 4, 8, 16), or 0 if none can.
inline int padded_group(int group) {
  for (int g = 1; g <= 16; g *= 2)
    if (group <= g) return g;
  return 0;
}

}  // namespace pagedkv
