// Launch parameters and kernel lookup of pa_multi_query and
// pa_decode_shared_prefix (multi_query.hip), shared by the kernels and their host
// code in multi_query_api.hip.  Internal.
#pragma once

#include "common.h"

namespace pagedkv {

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
  int log2_block_size;         // log2(block_size) for a power of two, else -1
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

}  // namespace pagedkv
