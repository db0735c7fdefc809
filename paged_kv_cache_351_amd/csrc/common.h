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
  float* ws_ml;        // [num_seqs][num_heads][max_parts] x {m, l}
  float* ws_acc;       // [num_seqs][num_heads][max_parts][head_dim]
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;           // num_heads / num_kv_heads
  int head_dim;
  int block_size;
  int num_blocks;
  int max_blocks_per_seq;
  int max_seq_len;
  int part_tokens;     // tokens per context partition
  int max_parts;       // ceil(max_seq_len / part_tokens), >= 1
  float scale_log2e;   // scale * log2(e): logits are taken in base 2
};

// Launchers, one translation unit per element type.  They return
// hipErrorInvalidValue for a shape outside the compiled set.
hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_f16(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream);

hipError_t launch_write_kv(const void* k, const void* v, const int32_t* slots,
                           void* k_cache, void* v_cache, int num_tokens,
                           int row_bytes, long long pool_slots, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int num_pairs, long long block_bytes, int num_blocks,
                              hipStream_t stream);

// Smallest group size of the compiled decode variants that can hold `group`
// query heads (1, 2, 4, 8, 16), or 0 if none can.
inline int padded_group(int group) {
  for (int g = 1; g <= 16; g *= 2)
    if (group <= g) return g;
  return 0;
}

}  // namespace pagedkv
