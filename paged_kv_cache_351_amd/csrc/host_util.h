// Host helpers shared by the C-ABI entry points of libpagedkv (validation,
// error text, debug checks).  Internal: not part of include/pagedkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "pagedkv.h"

namespace pagedkv {

constexpr int kMaxSeqLen = 1 << 24;   // longest sequence any entry point accepts

// Record a printf-style message for pa_last_error() on this thread; returns st.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status hip_fail(hipError_t e, const char* what);

// Positive integer value of an environment variable, else dflt.
int env_int(const char* name, int dflt);

// Environment switch: "0" is false, "1" true, anything else (or unset) dflt.
bool env_flag(const char* name, bool dflt);

// PA_DEBUG_CHECK=1: validate device-resident index data on the host before launching.
bool debug_checks();

inline bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Device address of ptr if the GPU may access it: device memory (returned as
// is) or pinned host memory mapped for the device.  Pageable host memory and
// unknown pointers give false; the query's error is cleared so that it does
// not surface in a later call.
bool device_address(const void* ptr, void** dev);

// Synchronous copy of n device elements to dst (PA_DEBUG_CHECK only).
template <typename T>
bool to_host(std::vector<T>& dst, const void* src, size_t n, hipStream_t stream, pa_status* st) {
  dst.resize(n);
  if (n == 0) return true;
  hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    *st = hip_fail(e, "PA_DEBUG_CHECK copy");
    return false;
  }
  return true;
}

}  // namespace pagedkv
