// C-ABI entry points of libpagedkv: argument validation, launch planning and
// dispatch.  The operations themselves are described in include/pagedkv.h.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "common.h"
#include "pagedkv.h"
#include "split.h"

using namespace pagedkv;

namespace {

thread_local std::string g_err;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

}  // namespace

void pagedkv::set_last_error(const char* msg) { g_err = msg; }

namespace {

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

bool debug_checks() {
  static const bool on = env_int("PA_DEBUG_CHECK", 0) == 1;
  return on;
}

// PA_DECODE_WAVES caps the number of decode waves (for tuning sweeps); 0 = no cap.
int requested_waves() {
  static const int v = env_int("PA_DECODE_WAVES", 0);
  return v;
}

// The last 1/12 of every wave's share goes to whichever wave is free first, in
// one part (smaller tails leave a longer finish, larger ones cost more chunk
// starts and partial results); PA_DECODE_TAIL = d overrides the divisor (0 = no tails) and
// PA_DECODE_TAIL_PIECES the number of parts (halving sizes), for tuning sweeps.
constexpr int kDefaultTailDiv = 12;
int tail_pieces() {
  static const int v = std::min(env_int("PA_DECODE_TAIL_PIECES", 1), kMaxTailPieces);
  return v;
}

int tail_divisor() {
  static const int v = [] {
    const char* s = getenv("PA_DECODE_TAIL");
    if (!s || !*s) return kDefaultTailDiv;
    char* end = nullptr;
    const long x = strtol(s, &end, 10);
    return (end && *end == 0 && x >= 0 && x <= 1024) ? (int)x : kDefaultTailDiv;
  }();
  return v;
}

bool valid_block_size(int bs) { return bs == 8 || bs == 16 || bs == 32; }

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Device address of ptr if the GPU may access it: device memory (returned as
// is) or pinned host memory mapped for the device.  Pageable host memory and
// unknown pointers give false; the query's error is cleared so that it does
// not surface in a later call.
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

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMaxSeqLen = 1 << 24;

// Workspace of one pa_decode call.  Each launched wave's share of the step is
// cut into chunks (a head and up to kMaxTailPieces tail parts); each chunk has
// a 16-byte record (the pair it owns, if split, and whether it left a first
// piece) and two partial-result slots (running max and sum, and the
// unnormalised accumulator, for each query head of the group).  A 256-byte header holds the chunk count and the counter
// that hands out tail chunks; the merge kernel leaves that counter at 0, so the
// workspace must be zero-filled before its first use only.  The size is the
// bound for the most waves the call could launch, which depends only on the
// shapes (one wave per kMinTilesPerWave tiles of the longest possible batch, at
// most kMaxWaves); the launch never uses more waves than that.
struct WorkspaceLayout {
  int waves;
  size_t ml_offset;
  size_t acc_offset;
  size_t total;
};

WorkspaceLayout plan_workspace(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                               int max_seq_len) {
  WorkspaceLayout w{0, 0, 0, 0};
  const long long t_max = (long long)num_seqs * num_kv_heads * tiles_of(max_seq_len);
  long long waves = waves_used(t_max, kMaxWaves);
  if (waves < 1) waves = 1;
  const size_t g = (size_t)(num_heads / num_kv_heads);
  const size_t chunks = (size_t)waves * (kMaxTailPieces + 1);
  const size_t slots = 2 * chunks;
  w.waves = (int)waves;
  w.ml_offset = align_up(256 + chunks * 16, 256);
  w.acc_offset = w.ml_offset + align_up(slots * g * 2 * sizeof(float), 256);
  w.total = w.acc_offset + slots * g * head_dim * sizeof(float);
  return w;
}

// Decode waves to launch on the current device: one per SIMD (4 per CU), or
// fewer if the kernel's occupancy does not allow that many at once; cached per
// device and kernel.  One wave per SIMD is deliberate: the SIMD issues its
// oldest wave first, so a second or third wave on it mostly waits for the
// first and then runs alone at the end; a single wave with two tiles in flight
// keeps HBM as busy and leaves no such tail.
hipError_t decode_waves(const void* kernel, int* out) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({dev, kernel});
  if (it != cache.end()) {
    *out = it->second;
    return hipSuccess;
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0);
  if (e != hipSuccess) return e;
  const int n = std::max(1, cus * std::min(per_cu, 1) * 4);
  cache[{dev, kernel}] = n;
  *out = n;
  return hipSuccess;
}

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

}  // namespace

extern "C" {

int pa_version(void) { return 6; }

const char* pa_last_error(void) { return g_err.c_str(); }

size_t pa_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                int max_seq_len) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_heads % num_kv_heads != 0 || max_seq_len < 0 || max_seq_len > kMaxSeqLen)
    return 0;
  return plan_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len).total;
}

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                    int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype dtype, void* out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_INVALID, "pa_decode: unknown dtype %d", (int)dtype);
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_seq_len < 0)
    return fail(PA_ERR_INVALID,
                "pa_decode: need num_seqs >= 0, num_heads, num_kv_heads, num_blocks, "
                "max_blocks_per_seq > 0 and max_seq_len >= 0");
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "pa_decode: num_heads (%d) is not a multiple of num_kv_heads (%d)",
                num_heads, num_kv_heads);
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
    return fail(PA_ERR_INVALID, "pa_decode: scale must be finite");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim %d not in {64, 128}", head_dim);
  if (!valid_block_size(block_size))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size %d not in {8, 16, 32}", block_size);
  const int group = num_heads / num_kv_heads;
  if (padded_group(group) == 0)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: %d query heads per KV head (at most 16)", group);
  if ((long long)max_seq_len > (long long)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID, "pa_decode: max_seq_len %d exceeds max_blocks_per_seq * block_size (%lld)",
                max_seq_len, (long long)max_blocks_per_seq * block_size);
  if (max_seq_len > kMaxSeqLen)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: max_seq_len %d above %d", max_seq_len, kMaxSeqLen);
  if ((long long)num_seqs * num_kv_heads * tiles_of(max_seq_len) >= (1LL << 40))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: batch of more than 2^40 tiles");
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
    return fail(PA_ERR_INVALID, "pa_decode: null pointer argument");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PA_ERR_INVALID, "pa_decode: q, caches and out must be 16-byte aligned");

  const WorkspaceLayout ws = plan_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len);
  if (!workspace || workspace_bytes < ws.total)
    return fail(PA_ERR_WORKSPACE, "pa_decode: workspace of %zu bytes needed, %zu given", ws.total,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(PA_ERR_WORKSPACE, "pa_decode: workspace must be 256-byte aligned");

  const void* dec = nullptr;
  const void* red = nullptr;
  const int gp = padded_group(group);
  bool found;
  switch (dtype) {
    case PA_F32: found = decode_kernels_f32(head_dim, block_size, gp, &dec, &red); break;
    case PA_F16: found = decode_kernels_f16(head_dim, block_size, gp, &dec, &red); break;
    default: found = decode_kernels_bf16(head_dim, block_size, gp, &dec, &red); break;
  }
  if (!found) return fail(PA_ERR_UNSUPPORTED, "pa_decode: no kernel for this shape");
  hipStream_t st = static_cast<hipStream_t>(stream);

  if (debug_checks()) {
    pa_status bad = PA_OK;
    std::vector<int32_t> lens, tab;
    if (!to_host(lens, seq_lens, num_seqs, st, &bad)) return bad;
    if (!to_host(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, st, &bad)) return bad;
    for (int s = 0; s < num_seqs; ++s) {
      if (lens[s] < 0 || lens[s] > max_seq_len)
        return fail(PA_ERR_INVALID, "pa_decode: seq_lens[%d] = %d outside [0, %d]", s, lens[s], max_seq_len);
      const int nb = (lens[s] + block_size - 1) / block_size;
      for (int j = 0; j < nb; ++j) {
        const int id = tab[(size_t)s * max_blocks_per_seq + j];
        if (id < 0 || id >= num_blocks)
          return fail(PA_ERR_INVALID, "pa_decode: block_tables[%d][%d] = %d outside [0, %d)", s, j, id,
                      num_blocks);
      }
    }
  }

  int waves = 0;
  hipError_t e = decode_waves(dec, &waves);
  if (e != hipSuccess) return hip_fail(e, "pa_decode occupancy query");
  waves = std::min(waves, ws.waves);
  if (requested_waves() > 0) waves = std::min(waves, requested_waves());

  DecodeParams p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.out = out;
  p.ws_meta = static_cast<int*>(workspace);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.ml_offset);
  p.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.acc_offset);
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.num_waves = waves;
  p.tail_div = tail_divisor();
  p.tail_pieces = tail_pieces();
  p.scale_log2e = (float)((double)scale * 1.4426950408889634074);

  void* kargs[] = {&p};
  // four waves per workgroup: one workgroup per CU, one wave per SIMD
  e = hipLaunchKernel(dec, dim3((waves + 3) / 4), dim3(256), kargs, 0, st);
  if (e != hipSuccess) return hip_fail(e, "pa_decode launch");
  // always: it also resets the tail counter for the next call
  e = hipLaunchKernel(red, dim3((waves * (p.tail_pieces + 1) + 3) / 4), dim3(256), kargs, 0, st);
  if (e != hipSuccess) return hip_fail(e, "pa_decode merge launch");
  return PA_OK;
}

namespace {

// Launch plan of pa_multi_query: a function of the shapes only, so that
// pa_multi_query_workspace_size and the launch agree.  Enough (sequence, KV head,
// query block, partition) items for about 1024 workgroups; partitions of at least
// 256 tokens, at most 64 of them.
struct MQPlan {
  int tq = 1, qblocks = 0, parts = 1;
  int rows = 64;               // query rows per workgroup (16: the waves split the context)
  bool split = false;
  size_t order_bytes = 0;      // longest-first item order at the head of the workspace
  long long items = 0;
  size_t ml_bytes = 0, total = 0;
};

constexpr int kMQMaxParts = 64;
constexpr long long kMQTargetItems = 1024;

MQPlan mq_plan(int num_seqs, int total_q, int num_heads, int num_kv_heads, int head_dim,
               int max_q_len, int max_seq_len, int dtype) {
  MQPlan pl;
  const int group = num_heads / num_kv_heads;
  pl.split = dtype != PA_F32 && max_q_len >= 1 && (long long)max_q_len * group <= 16;
  pl.rows = pl.split ? 16 : ((long long)max_q_len * group > 64 ? 128 : 64);
  pl.tq = pl.rows / group;
  pl.qblocks = max_q_len > 0 ? (max_q_len + pl.tq - 1) / pl.tq : 0;
  pl.items = (long long)num_seqs * num_kv_heads * pl.qblocks;
  if (pl.items > 0 && max_seq_len > 0) {
    const long long want = (kMQTargetItems + pl.items - 1) / pl.items;
    const long long by_len = ((long long)max_seq_len + 255) / 256;
    long long parts = want < by_len ? want : by_len;
    if (parts > kMQMaxParts) parts = kMQMaxParts;
    pl.parts = parts < 1 ? 1 : (int)parts;
  }
  // one query block per item (at most 16 rows): lengths alone set each item's work,
  // so the items are taken longest first
  if ((long long)max_q_len * group <= 16 && num_seqs > 0)
    pl.order_bytes = ((size_t)num_seqs * sizeof(int32_t) + 255) / 256 * 256;
  if (pl.parts > 1) {
    const size_t slots = (size_t)total_q * num_heads * pl.parts;
    pl.ml_bytes = (slots * 2 * sizeof(float) + 255) / 256 * 256;
    pl.total = pl.ml_bytes + slots * head_dim * sizeof(float);
  }
  pl.total += pl.order_bytes;
  return pl;
}

bool mq_shapes_ok(int num_seqs, int total_q, int num_heads, int num_kv_heads, int head_dim,
                  int max_q_len, int max_seq_len) {
  return num_seqs >= 0 && total_q >= 0 && num_heads > 0 && num_kv_heads > 0 && head_dim > 0 &&
         num_heads % num_kv_heads == 0 && num_heads / num_kv_heads <= 64 && max_q_len >= 0 && max_seq_len >= 0 &&
         max_seq_len <= kMaxSeqLen && max_q_len <= kMaxSeqLen;
}

}  // namespace

size_t pa_multi_query_workspace_size(int num_seqs, int total_q, int num_heads, int num_kv_heads,
                                     int head_dim, int max_q_len, int max_seq_len) {
  if (!mq_shapes_ok(num_seqs, total_q, num_heads, num_kv_heads, head_dim, max_q_len, max_seq_len))
    return 0;
  // the workspace does not depend on the element type (the split variant has one
  // query block whenever it applies, like the other)
  return mq_plan(num_seqs, total_q, num_heads, num_kv_heads, head_dim, max_q_len, max_seq_len, PA_BF16).total;
}

pa_status pa_multi_query(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* q_start, int num_seqs, int total_q, int num_heads,
                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                         int max_blocks_per_seq, int max_q_len, int max_seq_len, float scale,
                         pa_dtype dtype, void* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_INVALID, "pa_multi_query: unknown dtype %d", (int)dtype);
  if (num_seqs < 0 || total_q < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_q_len < 0 || max_seq_len < 0 || block_size <= 0)
    return fail(PA_ERR_INVALID,
                "pa_multi_query: need num_seqs, total_q, max_q_len, max_seq_len >= 0 and "
                "num_heads, num_kv_heads, block_size, num_blocks, max_blocks_per_seq > 0");
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "pa_multi_query: num_heads (%d) is not a multiple of num_kv_heads (%d)",
                num_heads, num_kv_heads);
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
    return fail(PA_ERR_INVALID, "pa_multi_query: scale must be finite");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_multi_query: head_dim %d not in {64, 128}", head_dim);
  if (num_heads / num_kv_heads > 64)
    return fail(PA_ERR_UNSUPPORTED, "pa_multi_query: %d query heads per KV head (at most 64)",
                num_heads / num_kv_heads);
  if ((long long)max_seq_len > (long long)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID, "pa_multi_query: max_seq_len %d exceeds max_blocks_per_seq * block_size (%lld)",
                max_seq_len, (long long)max_blocks_per_seq * block_size);
  if (max_seq_len > kMaxSeqLen || max_q_len > kMaxSeqLen)
    return fail(PA_ERR_UNSUPPORTED, "pa_multi_query: max_seq_len / max_q_len above %d", kMaxSeqLen);
  if (max_q_len > max_seq_len)
    return fail(PA_ERR_INVALID, "pa_multi_query: max_q_len %d above max_seq_len %d", max_q_len, max_seq_len);
  if ((long long)total_q * num_heads >= (1LL << 31))
    return fail(PA_ERR_UNSUPPORTED, "pa_multi_query: total_q * num_heads above 2^31");
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !q_start || !out)
    return fail(PA_ERR_INVALID, "pa_multi_query: null pointer argument");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PA_ERR_INVALID, "pa_multi_query: q, caches and out must be 16-byte aligned");
  const MQPlan pl = mq_plan(num_seqs, total_q, num_heads, num_kv_heads, head_dim, max_q_len, max_seq_len,
                            (int)dtype);
  if (pl.items * pl.parts + 8 >= (1LL << 31))
    return fail(PA_ERR_UNSUPPORTED, "pa_multi_query: more than 2^31 workgroups");
  if (pl.total > 0 && (!workspace || workspace_bytes < pl.total))
    return fail(PA_ERR_WORKSPACE, "pa_multi_query: workspace of %zu bytes, %zu needed", workspace_bytes,
                pl.total);
  if (pl.total > 0 && !aligned16(workspace))
    return fail(PA_ERR_INVALID, "pa_multi_query: workspace must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    pa_status bad = PA_OK;
    std::vector<int32_t> lens, qs, tab;
    if (!to_host(lens, seq_lens, num_seqs, st, &bad)) return bad;
    if (!to_host(qs, q_start, (size_t)num_seqs + 1, st, &bad)) return bad;
    if (!to_host(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, st, &bad)) return bad;
    if (qs[0] != 0 || qs[num_seqs] != total_q)
      return fail(PA_ERR_INVALID, "pa_multi_query: q_start must run from 0 to total_q");
    for (int s = 0; s < num_seqs; ++s) {
      const int n = qs[s + 1] - qs[s], L = lens[s];
      if (n < 0 || n > max_q_len)
        return fail(PA_ERR_INVALID, "pa_multi_query: sequence %d has %d queries (max_q_len %d)", s, n, max_q_len);
      if (L < 0 || L > max_seq_len || n > L)
        return fail(PA_ERR_INVALID, "pa_multi_query: sequence %d has length %d with %d queries", s, L, n);
      for (int j = 0; j < (L + block_size - 1) / block_size; ++j) {
        const int b = tab[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks)
          return fail(PA_ERR_INVALID, "pa_multi_query: block_tables[%d][%d] = %d outside [0, %d)", s, j, b,
                      num_blocks);
      }
    }
  }
  const void* kmain = nullptr;
  const void* kmerge = nullptr;
  if (!multi_query_kernels((int)dtype, head_dim, pl.rows, false, &kmain, &kmerge))
    return fail(PA_ERR_UNSUPPORTED, "pa_multi_query: no kernel for this dtype and head_dim");
  MultiQueryParams mp;
  mp.q = q;
  mp.k_cache = k_cache;
  mp.v_cache = v_cache;
  mp.block_tables = block_tables;
  mp.seq_lens = seq_lens;
  mp.q_start = q_start;
  mp.prefix_lens = nullptr;
  mp.out = out;
  char* ws = static_cast<char*>(workspace);
  mp.order = pl.order_bytes > 0 ? reinterpret_cast<const int32_t*>(ws) : nullptr;
  mp.order_out = pl.order_bytes > 0 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  mp.ws_ml = pl.parts > 1 ? reinterpret_cast<float*>(ws + pl.order_bytes) : nullptr;
  mp.ws_acc = pl.parts > 1 ? reinterpret_cast<float*>(ws + pl.order_bytes + pl.ml_bytes) : nullptr;
  mp.num_seqs = num_seqs;
  mp.total_q = total_q;
  mp.num_heads = num_heads;
  mp.num_kv_heads = num_kv_heads;
  mp.group = num_heads / num_kv_heads;
  mp.head_dim = head_dim;
  mp.block_size = block_size;
  mp.inv_block_size = 1.0f / (float)block_size;
  mp.num_blocks = num_blocks;
  mp.max_blocks_per_seq = max_blocks_per_seq;
  mp.max_q_len = max_q_len;
  mp.max_seq_len = max_seq_len;
  mp.tq = pl.tq;
  mp.qblocks = pl.qblocks;
  mp.parts = pl.parts;
  mp.items = pl.items;
  mp.scale_log2e = (float)((double)scale * 1.4426950408889634074);
  const long long wgs = (pl.items * pl.parts + 7) / 8 * 8;
  void* args[] = {&mp};
  hipError_t e;
  if (pl.order_bytes > 0) {
    e = hipLaunchKernel(multi_query_order_kernel(false), dim3(1), dim3(1024), args, 0, st);
    if (e != hipSuccess) return hip_fail(e, "pa_multi_query order launch");
  }
  e = hipLaunchKernel(kmain, dim3((unsigned)wgs), dim3(256), args, 0, st);
  if (e != hipSuccess) return hip_fail(e, "pa_multi_query launch");
  if (pl.parts > 1) {
    const long long rows = (long long)total_q * num_heads;
    e = hipLaunchKernel(kmerge, dim3((unsigned)((rows + 3) / 4)), dim3(256), args, 0, st);
    if (e != hipSuccess) return hip_fail(e, "pa_multi_query merge launch");
  }
  return PA_OK;
}

namespace {

// Launch plan of pa_decode_shared_prefix: items are (group, KV head, block of
// 16 / group members); otherwise as for pa_multi_query.
MQPlan sp_plan(int num_seqs, int num_groups, int num_heads, int num_kv_heads, int head_dim,
               int max_group_size, int max_seq_len) {
  MQPlan pl;
  const int group = num_heads / num_kv_heads;
  pl.split = true;
  pl.rows = 16;
  pl.tq = 16 / group;
  pl.qblocks = max_group_size > 0 ? (max_group_size + pl.tq - 1) / pl.tq : 0;
  pl.items = (long long)num_groups * num_kv_heads * pl.qblocks;
  if (pl.items > 0 && max_seq_len > 0) {
    const long long want = (kMQTargetItems + pl.items - 1) / pl.items;
    const long long by_len = ((long long)max_seq_len + 255) / 256;
    long long parts = want < by_len ? want : by_len;
    if (parts > kMQMaxParts) parts = kMQMaxParts;
    pl.parts = parts < 1 ? 1 : (int)parts;
  }
  if (num_groups > 0) pl.order_bytes = ((size_t)num_groups * sizeof(int32_t) + 255) / 256 * 256;
  if (pl.parts > 1) {
    const size_t slots = (size_t)num_seqs * num_heads * pl.parts;
    pl.ml_bytes = (slots * 2 * sizeof(float) + 255) / 256 * 256;
    pl.total = pl.ml_bytes + slots * head_dim * sizeof(float);
  }
  pl.total += pl.order_bytes;
  return pl;
}

}  // namespace

size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int num_groups, int num_heads,
                                              int num_kv_heads, int head_dim, int max_group_size,
                                              int max_seq_len) {
  if (num_seqs < 0 || num_groups < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_heads % num_kv_heads != 0 || num_heads / num_kv_heads > 16 || max_group_size < 0 ||
      max_seq_len < 0 || max_seq_len > kMaxSeqLen)
    return 0;
  return sp_plan(num_seqs, num_groups, num_heads, num_kv_heads, head_dim, max_group_size, max_seq_len).total;
}

pa_status pa_decode_shared_prefix(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens,
                                  int num_seqs, int num_groups, int num_heads, int num_kv_heads,
                                  int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_group_size, int max_seq_len, float scale, pa_dtype dtype,
                                  void* out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "pa_decode_shared_prefix";
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_INVALID, "%s: unknown dtype %d", who, (int)dtype);
  if (num_seqs < 0 || num_groups < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_group_size < 0 || max_seq_len < 0 || block_size <= 0)
    return fail(PA_ERR_INVALID,
                "%s: need num_seqs, num_groups, max_group_size, max_seq_len >= 0 and num_heads, "
                "num_kv_heads, block_size, num_blocks, max_blocks_per_seq > 0", who);
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "%s: num_heads (%d) is not a multiple of num_kv_heads (%d)", who,
                num_heads, num_kv_heads);
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
    return fail(PA_ERR_INVALID, "%s: scale must be finite", who);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", who, head_dim);
  if (dtype == PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "%s: float32 caches are not supported (use pa_decode)", who);
  if (num_heads / num_kv_heads > 16)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d query heads per KV head (at most 16)", who,
                num_heads / num_kv_heads);
  if ((long long)max_seq_len > (long long)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID, "%s: max_seq_len %d exceeds max_blocks_per_seq * block_size (%lld)", who,
                max_seq_len, (long long)max_blocks_per_seq * block_size);
  if (max_seq_len > kMaxSeqLen)
    return fail(PA_ERR_UNSUPPORTED, "%s: max_seq_len %d above %d", who, max_seq_len, kMaxSeqLen);
  if (max_group_size > num_seqs)
    return fail(PA_ERR_INVALID, "%s: max_group_size %d above num_seqs %d", who, max_group_size, num_seqs);
  if ((long long)num_seqs * num_heads >= (1LL << 31))
    return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs * num_heads above 2^31", who);
  if (num_seqs == 0 || num_groups == 0 || max_group_size == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !group_start || !prefix_lens || !out)
    return fail(PA_ERR_INVALID, "%s: null pointer argument", who);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PA_ERR_INVALID, "%s: q, caches and out must be 16-byte aligned", who);
  const MQPlan pl = sp_plan(num_seqs, num_groups, num_heads, num_kv_heads, head_dim, max_group_size,
                            max_seq_len);
  if (pl.items * pl.parts + 8 >= (1LL << 31))
    return fail(PA_ERR_UNSUPPORTED, "%s: more than 2^31 workgroups", who);
  if (pl.total > 0 && (!workspace || workspace_bytes < pl.total))
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes, pl.total);
  if (pl.total > 0 && !aligned16(workspace))
    return fail(PA_ERR_INVALID, "%s: workspace must be 16-byte aligned", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    pa_status bad = PA_OK;
    std::vector<int32_t> lens, gs, pre, tab;
    if (!to_host(lens, seq_lens, num_seqs, st, &bad)) return bad;
    if (!to_host(gs, group_start, (size_t)num_groups + 1, st, &bad)) return bad;
    if (!to_host(pre, prefix_lens, num_groups, st, &bad)) return bad;
    if (!to_host(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, st, &bad)) return bad;
    if (gs[0] != 0 || gs[num_groups] != num_seqs)
      return fail(PA_ERR_INVALID, "%s: group_start must run from 0 to num_seqs", who);
    for (int s = 0; s < num_seqs; ++s) {
      if (lens[s] < 0 || lens[s] > max_seq_len)
        return fail(PA_ERR_INVALID, "%s: seq_lens[%d] = %d outside [0, %d]", who, s, lens[s], max_seq_len);
      for (int j = 0; j < (lens[s] + block_size - 1) / block_size; ++j) {
        const int b = tab[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks)
          return fail(PA_ERR_INVALID, "%s: block_tables[%d][%d] = %d outside [0, %d)", who, s, j, b, num_blocks);
      }
    }
    for (int gi = 0; gi < num_groups; ++gi) {
      const int a = gs[gi], b = gs[gi + 1];
      if (b < a || b - a > max_group_size)
        return fail(PA_ERR_INVALID, "%s: group %d has %d members (max_group_size %d)", who, gi, b - a,
                    max_group_size);
      const int P = pre[gi];
      for (int s = a; s < b; ++s) {
        if (P < 0 || P > lens[s])
          return fail(PA_ERR_INVALID, "%s: prefix_lens[%d] = %d not within sequence %d's %d tokens", who,
                      gi, P, s, lens[s]);
        for (int j = 0; j < (P + block_size - 1) / block_size; ++j)
          if (tab[(size_t)s * max_blocks_per_seq + j] != tab[(size_t)a * max_blocks_per_seq + j])
            return fail(PA_ERR_INVALID, "%s: sequence %d does not share block %d of group %d's prefix", who,
                        s, j, gi);
      }
    }
  }
  const void* kmain = nullptr;
  const void* kmerge = nullptr;
  if (!multi_query_kernels((int)dtype, head_dim, 16, true, &kmain, &kmerge))
    return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for this dtype and head_dim", who);
  MultiQueryParams mp;
  mp.q = q;
  mp.k_cache = k_cache;
  mp.v_cache = v_cache;
  mp.block_tables = block_tables;
  mp.seq_lens = seq_lens;
  mp.q_start = group_start;
  mp.prefix_lens = prefix_lens;
  mp.out = out;
  char* ws = static_cast<char*>(workspace);
  mp.order = pl.order_bytes > 0 ? reinterpret_cast<const int32_t*>(ws) : nullptr;
  mp.order_out = pl.order_bytes > 0 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  mp.ws_ml = pl.parts > 1 ? reinterpret_cast<float*>(ws + pl.order_bytes) : nullptr;
  mp.ws_acc = pl.parts > 1 ? reinterpret_cast<float*>(ws + pl.order_bytes + pl.ml_bytes) : nullptr;
  mp.num_seqs = num_groups;          // items run over groups
  mp.total_q = num_seqs;             // rows are member sequences
  mp.num_heads = num_heads;
  mp.num_kv_heads = num_kv_heads;
  mp.group = num_heads / num_kv_heads;
  mp.head_dim = head_dim;
  mp.block_size = block_size;
  mp.inv_block_size = 1.0f / (float)block_size;
  mp.num_blocks = num_blocks;
  mp.max_blocks_per_seq = max_blocks_per_seq;
  mp.max_q_len = max_group_size;
  mp.max_seq_len = max_seq_len;
  mp.tq = pl.tq;
  mp.qblocks = pl.qblocks;
  mp.parts = pl.parts;
  mp.items = pl.items;
  mp.scale_log2e = (float)((double)scale * 1.4426950408889634074);
  const long long wgs = (pl.items * pl.parts + 7) / 8 * 8;
  void* args[] = {&mp};
  hipError_t e = hipLaunchKernel(multi_query_order_kernel(true), dim3(1), dim3(1024), args, 0, st);
  if (e != hipSuccess) return hip_fail(e, "pa_decode_shared_prefix order launch");
  e = hipLaunchKernel(kmain, dim3((unsigned)wgs), dim3(256), args, 0, st);
  if (e != hipSuccess) return hip_fail(e, "pa_decode_shared_prefix launch");
  if (pl.parts > 1) {
    const long long rows = (long long)num_seqs * num_heads;
    e = hipLaunchKernel(kmerge, dim3((unsigned)((rows + 3) / 4)), dim3(256), args, 0, st);
    if (e != hipSuccess) return hip_fail(e, "pa_decode_shared_prefix merge launch");
  }
  return PA_OK;
}

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
