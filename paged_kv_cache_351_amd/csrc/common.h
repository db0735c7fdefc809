// Internal declarations shared by the HIP kernels and the C-ABI host code of
// libpagedkv.  Not part of the public interface (that is include/pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pagedkv {

enum ElemType { kF32 = 0, kF16 = 1, kBF16 = 2 };

inline int elem_bytes(int dt) { return dt == kF32 ? 4 : 2; }

hipError_t launch_write_kv(const void* k, const void* v, const int32_t* slots,
                           void* k_cache, void* v_cache, int num_tokens,
                           int row_bytes, long long pool_slots, hipStream_t stream);

hipError_t launch_copy_blocks(const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                              const int32_t* pairs, int num_pairs, long long block_bytes,
                              int src_blocks, int dst_blocks, hipStream_t stream);

// Message returned by pa_last_error() on the calling thread.
void set_last_error(const char* msg);

}  // namespace pagedkv
