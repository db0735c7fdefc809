// pa_decode and pa_decode_workspace_size: validation, workspace layout and the
// launch plan of the decode and merge kernels (decode_kernel.h, split.h).
#include <stdlib.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "decode_params.h"
#include "host_util.h"
#include "pagedkv.h"
#include "split.h"

using namespace pagedkv;

namespace {

// PA_DECODE_WAVES caps the number of decode waves (for tuning sweeps); 0 = no cap.
int requested_waves() {
  static const int v = env_int("PA_DECODE_WAVES", 0);
  return v;
}

// The last 1/16 of every wave's share goes to whichever wave is free first, in
// one part (smaller tails leave a longer finish, larger ones cost more chunk
// starts and partial results); with short shares the kernel lowers the divisor so a
// part keeps at least 16 tiles (split.h, effective_tail_div), down to 1/8.
// PA_DECODE_TAIL = d overrides the divisor (0 = no tails) and
// PA_DECODE_TAIL_PIECES the number of parts (halving sizes), for tuning sweeps.
constexpr int kDefaultTailDiv = 16;
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

}  // namespace

extern "C" {

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

}  // extern "C"
