// KV write (slot append) and block copy (copy-on-write) kernels.  Both only move
// bits, 16 bytes per lane per access, so they are bound by HBM bandwidth and
// launch latency.
//
// Write: a new token's K/V goes to the next free slot of its sequence's last
// block; the host has already turned that into a flat slot index per token
// ("LLM 注意力与计算内核精读笔记 · 05 PagedAttention 与 KV 显存管理", §5 ②).
// Copy: before writing into a block other sequences still share, the writer's
// block is duplicated (same page, §6.1 and §12 题4).
// Swap: a preempted request's blocks move to CPU RAM and back (same page, §5 ③);
// the same block copy, between two pools.
#include "common.h"

namespace pagedkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// grid.x = token, grid.y strides over the 2 * row_vec 16-byte pieces of its K and V rows.
__global__ __launch_bounds__(256) void write_kv_kernel(const u32x4* __restrict__ k,
                                                        const u32x4* __restrict__ v,
                                                        const int32_t* __restrict__ slots,
                                                        u32x4* __restrict__ k_cache,
                                                        u32x4* __restrict__ v_cache, int row_vec,
                                                        long long pool_slots) {
  const int tok = blockIdx.x;
  const int slot = slots[tok];
  if (slot < 0 || (long long)slot >= pool_slots) return;
  const size_t src = (size_t)tok * row_vec;
  const size_t dst = (size_t)slot * row_vec;
  for (int i = blockIdx.y * 256 + threadIdx.x; i < 2 * row_vec; i += gridDim.y * 256) {
    if (i < row_vec) {
      k_cache[dst + i] = k[src + i];
    } else {
      v_cache[dst + i - row_vec] = v[src + i - row_vec];
    }
  }
}

// grid.x = pair, grid.y = 1024-piece chunk of the block; each lane moves four
// 16-byte pieces of K and four of V, loads first.  Source and destination pools
// may be the same (copy-on-write) or two different pools (swap between HBM and
// pinned host memory, which the GPU reads and writes over the host link).
__global__ __launch_bounds__(256) void copy_blocks_kernel(const u32x4* ksrc, const u32x4* vsrc,
                                                           u32x4* kdst, u32x4* vdst,
                                                           const int32_t* __restrict__ pairs,
                                                           int src_blocks, int dst_blocks,
                                                           long long blk_vec) {
  const int src = pairs[2 * blockIdx.x];
  const int dst = pairs[2 * blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)src_blocks || (unsigned)dst >= (unsigned)dst_blocks) return;
  const long long base = (long long)blockIdx.y * 1024 + threadIdx.x;
  const u32x4* ks = ksrc + (size_t)src * blk_vec;
  const u32x4* vs = vsrc + (size_t)src * blk_vec;
  u32x4* kd = kdst + (size_t)dst * blk_vec;
  u32x4* vd = vdst + (size_t)dst * blk_vec;
  u32x4 a[4], b[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const long long i = base + u * 256;
    if (i < blk_vec) {
      a[u] = ks[i];
      b[u] = vs[i];
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const long long i = base + u * 256;
    if (i < blk_vec) {
      kd[i] = a[u];
      vd[i] = b[u];
    }
  }
}

hipError_t launch_write_kv(const void* k, const void* v, const int32_t* slots, void* k_cache,
                           void* v_cache, int num_tokens, int row_bytes, long long pool_slots,
                           hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  int row_vec = row_bytes / 16;
  const int chunks = (2 * row_vec + 255) / 256;
  const u32x4* kk = static_cast<const u32x4*>(k);
  const u32x4* vv = static_cast<const u32x4*>(v);
  u32x4* kc = static_cast<u32x4*>(k_cache);
  u32x4* vc = static_cast<u32x4*>(v_cache);
  void* args[] = {&kk, &vv, &slots, &kc, &vc, &row_vec, &pool_slots};
  return hipLaunchKernel(reinterpret_cast<const void*>(&write_kv_kernel), dim3(num_tokens, chunks),
                         dim3(256), args, 0, stream);
}

hipError_t launch_copy_blocks(const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                              const int32_t* pairs, int num_pairs, long long block_bytes,
                              int src_blocks, int dst_blocks, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  long long blk_vec = block_bytes / 16;
  const long long chunks = (blk_vec + 1023) / 1024;
  const u32x4* ks = static_cast<const u32x4*>(k_src);
  const u32x4* vs = static_cast<const u32x4*>(v_src);
  u32x4* kd = static_cast<u32x4*>(k_dst);
  u32x4* vd = static_cast<u32x4*>(v_dst);
  void* args[] = {&ks, &vs, &kd, &vd, &pairs, &src_blocks, &dst_blocks, &blk_vec};
  return hipLaunchKernel(reinterpret_cast<const void*>(&copy_blocks_kernel),
                         dim3(num_pairs, (unsigned)chunks), dim3(256), args, 0, stream);
}

}  // namespace pagedkv
