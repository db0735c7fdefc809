// C-ABI entry points of libpagedkv shared by every path: version, error text,
// the KV write, block copy and swap.  pa_decode is in decode_api.hip, the
// multi-query and shared-prefix calls in multi_query_api.hip; block_manager.hip
// holds the host block manager.  The operations are described in
// include/pagedkv.h.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <string>
#include <vector>

#include "common.h"
#include "host_util.h"
#include "pagedkv.h"

namespace {

thread_local std::string g_err;

}  // namespace

namespace pagedkv {

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

void set_last_error(const char* msg) { g_err = msg; }

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  char* end = nullptr;
  long v = strtol(s, &end, 10);
  return (end && *end == 0 && v > 0 && v < (1L << 30)) ? (int)v : dflt;
}

bool env_flag(const char* name, bool dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  if (s[0] == '0' && s[1] == 0) return false;
  if (s[0] == '1' && s[1] == 0) return true;
  return dflt;
}

bool debug_checks() {
  static const bool on = env_int("PA_DEBUG_CHECK", 0) == 1;
  return on;
}

bool device_address(const void* ptr, void** dev) {
  hipPointerAttribute_t a;
  const hipError_t e = hipPointerGetAttributes(&a, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
    *dev = const_cast<void*>(ptr);
    return true;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer != nullptr) {
    *dev = a.devicePointer;
    return true;
  }
  return false;
}

}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

int pa_version(void) { return 9; }

const char* pa_last_error(void) { return g_err.c_str(); }

pa_status pa_write_kv(const void* k, const void* v, const int32_t* slot_mapping, void* k_cache,
                      void* v_cache, int num_tokens, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, pa_dtype dtype, void* stream) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_INVALID, "pa_write_kv: unknown dtype %d", (int)dtype);
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID, "pa_write_kv: need num_tokens >= 0 and positive sizes");
  const long long row_bytes = (long long)num_kv_heads * head_dim * elem_bytes(dtype);
  if (row_bytes % 16 != 0 || row_bytes / 16 > (1 << 22))
    return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: a token row of %lld bytes is not a multiple of 16 "
                "bytes or exceeds 64 MiB", row_bytes);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID, "pa_write_kv: null pointer argument");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID, "pa_write_kv: k, v and caches must be 16-byte aligned");
  const long long pool_slots = (long long)num_blocks * block_size;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    pa_status bad = PA_OK;
    std::vector<int32_t> slots;
    if (!to_host(slots, slot_mapping, num_tokens, st, &bad)) return bad;
    std::vector<int32_t> live;
    for (int i = 0; i < num_tokens; ++i) {
      if (slots[i] >= pool_slots)
        return fail(PA_ERR_INVALID, "pa_write_kv: slot_mapping[%d] = %d beyond the pool", i, slots[i]);
      if (slots[i] >= 0) live.push_back(slots[i]);
    }
    std::sort(live.begin(), live.end());
    for (size_t i = 1; i < live.size(); ++i)
      if (live[i] == live[i - 1]) return fail(PA_ERR_INVALID, "pa_write_kv: slot %d named twice", live[i]);
  }
  hipError_t e = launch_write_kv(k, v, slot_mapping, k_cache, v_cache, num_tokens, (int)row_bytes,
                                 pool_slots, st);
  if (e != hipSuccess) return hip_fail(e, "pa_write_kv launch");
  return PA_OK;
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst_pairs, int num_pairs,
                         int block_size, int num_kv_heads, int head_dim, int num_blocks,
                         pa_dtype dtype, void* stream) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_INVALID, "pa_copy_blocks: unknown dtype %d", (int)dtype);
  if (num_pairs < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID, "pa_copy_blocks: need num_pairs >= 0 and positive sizes");
  const long long block_bytes = (long long)block_size * num_kv_heads * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0 || block_bytes / 16 > 65535LL * 1024)
    return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: a block of %lld bytes is not a multiple of 16 "
                "bytes or exceeds 1 GiB", block_bytes);
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_dst_pairs)
    return fail(PA_ERR_INVALID, "pa_copy_blocks: null pointer argument");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID, "pa_copy_blocks: caches must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    pa_status bad = PA_OK;
    std::vector<int32_t> pr;
    if (!to_host(pr, src_dst_pairs, (size_t)num_pairs * 2, st, &bad)) return bad;
    std::vector<int32_t> srcs, dsts;
    for (int i = 0; i < num_pairs; ++i) {
      const int s = pr[2 * i], d = pr[2 * i + 1];
      if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
        return fail(PA_ERR_INVALID, "pa_copy_blocks: pair %d (%d, %d) outside [0, %d)", i, s, d, num_blocks);
      if (s == d) return fail(PA_ERR_INVALID, "pa_copy_blocks: pair %d copies block %d onto itself", i, s);
      srcs.push_back(s);
      dsts.push_back(d);
    }
    std::sort(srcs.begin(), srcs.end());
    std::sort(dsts.begin(), dsts.end());
    for (size_t i = 1; i < dsts.size(); ++i)
      if (dsts[i] == dsts[i - 1]) return fail(PA_ERR_INVALID, "pa_copy_blocks: dst %d repeated", dsts[i]);
    for (int d : dsts)
      if (std::binary_search(srcs.begin(), srcs.end(), d))
        return fail(PA_ERR_INVALID, "pa_copy_blocks: block %d is both a src and a dst", d);
  }
  hipError_t e = launch_copy_blocks(k_cache, v_cache, k_cache, v_cache, src_dst_pairs, num_pairs,
                                    block_bytes, num_blocks, num_blocks, st);
  if (e != hipSuccess) return hip_fail(e, "pa_copy_blocks launch");
  return PA_OK;
}

pa_status pa_swap_blocks(const void* src_k, const void* src_v, int src_num_blocks, void* dst_k,
                         void* dst_v, int dst_num_blocks, const int32_t* src_dst_pairs,
                         int num_pairs, int block_size, int num_kv_heads, int head_dim,
                         pa_dtype dtype, void* stream) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_INVALID, "pa_swap_blocks: unknown dtype %d", (int)dtype);
  if (num_pairs < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      src_num_blocks <= 0 || dst_num_blocks <= 0)
    return fail(PA_ERR_INVALID, "pa_swap_blocks: need num_pairs >= 0 and positive sizes");
  const long long block_bytes = (long long)block_size * num_kv_heads * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0 || block_bytes / 16 > 65535LL * 1024)
    return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: a block of %lld bytes is not a multiple of 16 "
                "bytes or exceeds 1 GiB", block_bytes);
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !src_dst_pairs)
    return fail(PA_ERR_INVALID, "pa_swap_blocks: null pointer argument");
  if (src_k == dst_k || src_v == dst_v)
    return fail(PA_ERR_INVALID, "pa_swap_blocks: source and destination are the same pool "
                "(use pa_copy_blocks)");
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
    return fail(PA_ERR_INVALID, "pa_swap_blocks: pools must be 16-byte aligned");
  // Every array the kernel touches must be device memory or pinned host memory
  // mapped for the device; a pageable host pointer is refused here rather than
  // faulting in the kernel.
  const void* in[5] = {src_k, src_v, dst_k, dst_v, src_dst_pairs};
  const char* name[5] = {"src_k", "src_v", "dst_k", "dst_v", "src_dst_pairs"};
  void* dev[5];
  for (int i = 0; i < 5; ++i) {
    if (!device_address(in[i], &dev[i]))
      return fail(PA_ERR_INVALID, "pa_swap_blocks: %s is neither device memory nor pinned host "
                  "memory mapped for the device", name[i]);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    pa_status bad = PA_OK;
    std::vector<int32_t> pr;
    if (!to_host(pr, src_dst_pairs, (size_t)num_pairs * 2, st, &bad)) return bad;
    std::vector<int32_t> dsts;
    for (int i = 0; i < num_pairs; ++i) {
      const int s = pr[2 * i], d = pr[2 * i + 1];
      if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks)
        return fail(PA_ERR_INVALID, "pa_swap_blocks: pair %d (%d, %d) outside the pools", i, s, d);
      dsts.push_back(d);
    }
    std::sort(dsts.begin(), dsts.end());
    for (size_t i = 1; i < dsts.size(); ++i)
      if (dsts[i] == dsts[i - 1]) return fail(PA_ERR_INVALID, "pa_swap_blocks: dst %d repeated", dsts[i]);
  }
  hipError_t e = launch_copy_blocks(dev[0], dev[1], dev[2], dev[3],
                                    static_cast<const int32_t*>(dev[4]), num_pairs, block_bytes,
                                    src_num_blocks, dst_num_blocks, st);
  if (e != hipSuccess) return hip_fail(e, "pa_swap_blocks launch");
  return PA_OK;
}

}  // extern "C"
