// pa_decode, pa_decode_cached, pa_decode_append and pa_decode_workspace_size: validation,
// workspace layout and the launch plan of the decode and merge kernels (decode_kernel.h,
// split.h).
#include <stdlib.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <unordered_map>
#include <unordered_set>
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

// The multi-query rows mode hands out no tail parts by default: its pieces carry up to 16
// rows, and the fewer pieces of a static split (two per wave rather than about three)
// cost less than the longer finish (Llama-3-8B verification: 439 against 445 us for
// 1/16 tails).  PA_MULTI_QUERY_ROWS_TAIL = d sets a divisor, for tuning sweeps.
int rows_tail_divisor() {
  static const int v = std::max(0, std::min(env_int("PA_MULTI_QUERY_ROWS_TAIL", 0), 1024));
  return v;
}

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

WorkspaceLayout layout_for(long long waves, int pieces, int group, int head_dim) {
  WorkspaceLayout w{0, 0, 0, 0};
  if (waves < 1) waves = 1;
  const size_t g = (size_t)group;
  const size_t chunks = (size_t)waves * (pieces + 1);
  const size_t slots = 2 * chunks;
  w.waves = (int)waves;
  w.ml_offset = align_up(256 + chunks * 16, 256);
  w.acc_offset = w.ml_offset + align_up(slots * g * 2 * sizeof(float), 256);
  w.total = w.acc_offset + slots * g * head_dim * sizeof(float);
  return w;
}

WorkspaceLayout plan_workspace(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                               int max_seq_len) {
  const long long t_max = (long long)num_seqs * num_kv_heads * tiles_of(max_seq_len);
  return layout_for(waves_used(t_max, kMaxWaves), kMaxTailPieces, num_heads / num_kv_heads, head_dim);
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

}  // extern "C"

// ---------------------------------------------------------------------------------
// The decode path for callers that cannot allocate.  Its workspace is this file-scope
// device array: every GPU the library runs on holds its own copy, at its own address,
// until the process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: host code uses only the address hipGetSymbolAddress returns for
// the current device.
static __device__ __align__(256) char scratch[PA_DECODE_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kNoAllocScratchBytes = PA_DECODE_NO_ALLOC_SCRATCH_BYTES;

// With debug checks on, for pa_decode_append: every sequence's newest slot (position
// seq_lens[s] - 1) belongs to it alone.  No two sequences append into one slot, and no
// other (sequence, position) of the batch reads it, so the write needs no ordering
// against the reads of other waves.  The ids are already known to be in the pool.
pa_status check_append_slots(const std::vector<int32_t>& lens, const std::vector<int32_t>& tab,
                             int num_seqs, int block_size, int max_blocks_per_seq, const char* who) {
  std::unordered_map<long long, int> owner;  // appended slot -> its sequence
  std::unordered_set<int> blocks;            // blocks holding an appended slot
  for (int s = 0; s < num_seqs; ++s) {
    if (lens[s] == 0) continue;
    const int t = lens[s] - 1;
    const int id = tab[(size_t)s * max_blocks_per_seq + t / block_size];
    const long long slot = (long long)id * block_size + t % block_size;
    auto ins = owner.emplace(slot, s);
    if (!ins.second)
      return fail(PA_ERR_INVALID, "%s: sequences %d and %d both append into slot %lld", who,
                  ins.first->second, s, slot);
    blocks.insert(id);
  }
  for (int s = 0; s < num_seqs; ++s) {
    const int nb = (lens[s] + block_size - 1) / block_size;
    for (int j = 0; j < nb; ++j) {
      const int id = tab[(size_t)s * max_blocks_per_seq + j];
      if (blocks.count(id) == 0) continue;
      for (int t = j * block_size; t < std::min(lens[s], (j + 1) * block_size); ++t) {
        auto it = owner.find((long long)id * block_size + t % block_size);
        if (it != owner.end() && !(it->second == s && t == lens[s] - 1))
          return fail(PA_ERR_INVALID,
                      "%s: slot %lld, appended by sequence %d, is also read by sequence %d at "
                      "position %d", who, it->first, it->second, s, t);
      }
    }
  }
  return PA_OK;
}

// Everything pa_decode, pa_decode_cached, pa_decode_append and pa_decode_no_alloc share:
// argument checks, the kernels, the debug checks of the index data and the launch
// parameters (DecodeParams without the workspace pointers).  new_k and new_v are null
// except for pa_decode_append (variant kAppend).  Returns PA_OK with *skip set when there is nothing to launch.
pa_status prepare_decode(DecodeVariant variant, const void* q, const void* k_cache,
                         const void* v_cache, const void* new_k, const void* new_v,
                         const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                         int num_heads, int num_kv_heads, int head_dim, int block_size,
                         int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                         pa_dtype dtype, void* out, hipStream_t st, const char* who,
                         const void* workspace, size_t workspace_bytes, bool check_workspace,
                         DecodeParams* p, const void** dec, const void** red, bool* skip) {
  *skip = false;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_INVALID, "%s: unknown dtype %d", who, (int)dtype);
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_seq_len < 0)
    return fail(PA_ERR_INVALID,
                "%s: need num_seqs >= 0, num_heads, num_kv_heads, num_blocks, "
                "max_blocks_per_seq > 0 and max_seq_len >= 0", who);
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "%s: num_heads (%d) is not a multiple of num_kv_heads (%d)", who,
                num_heads, num_kv_heads);
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
    return fail(PA_ERR_INVALID, "%s: scale must be finite", who);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", who, head_dim);
  if (!valid_block_size(block_size))
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d not in {8, 16, 32}", who, block_size);
  const int group = num_heads / num_kv_heads;
  if (padded_group(group) == 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d query heads per KV head (at most 16)", who, group);
  if ((long long)max_seq_len > (long long)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID, "%s: max_seq_len %d exceeds max_blocks_per_seq * block_size (%lld)",
                who, max_seq_len, (long long)max_blocks_per_seq * block_size);
  if (max_seq_len > kMaxSeqLen)
    return fail(PA_ERR_UNSUPPORTED, "%s: max_seq_len %d above %d", who, max_seq_len, kMaxSeqLen);
  if ((long long)num_seqs * num_kv_heads * tiles_of(max_seq_len) >= (1LL << 40))
    return fail(PA_ERR_UNSUPPORTED, "%s: batch of more than 2^40 tiles", who);
  if (num_seqs == 0) {
    *skip = true;
    return PA_OK;
  }
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
    return fail(PA_ERR_INVALID, "%s: null pointer argument", who);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PA_ERR_INVALID, "%s: q, caches and out must be 16-byte aligned", who);
  if ((new_k == nullptr) != (new_v == nullptr))
    return fail(PA_ERR_INVALID, "%s: new_k and new_v must both be given", who);
  if (new_k && (!aligned16(new_k) || !aligned16(new_v)))
    return fail(PA_ERR_INVALID, "%s: new_k and new_v must be 16-byte aligned", who);
  if (check_workspace) {
    const WorkspaceLayout ws = plan_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len);
    if (!workspace || workspace_bytes < ws.total)
      return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, ws.total,
                  workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(PA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", who);
  }

  const int gp = variant == DecodeVariant::kRows ? 16 : padded_group(group);
  bool found;
  switch (dtype) {
    case PA_F32: found = decode_kernels_f32(head_dim, block_size, gp, variant, dec, red); break;
    case PA_F16: found = decode_kernels_f16(head_dim, block_size, gp, variant, dec, red); break;
    default: found = decode_kernels_bf16(head_dim, block_size, gp, variant, dec, red); break;
  }
  if (!found) return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for this shape", who);

  if (debug_checks()) {
    pa_status bad = PA_OK;
    std::vector<int32_t> lens, tab;
    if (!to_host(lens, seq_lens, num_seqs, st, &bad)) return bad;
    if (!to_host(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, st, &bad)) return bad;
    for (int s = 0; s < num_seqs; ++s) {
      if (lens[s] < 0 || lens[s] > max_seq_len)
        return fail(PA_ERR_INVALID, "%s: seq_lens[%d] = %d outside [0, %d]", who, s, lens[s],
                    max_seq_len);
      const int nb = (lens[s] + block_size - 1) / block_size;
      for (int j = 0; j < nb; ++j) {
        const int id = tab[(size_t)s * max_blocks_per_seq + j];
        if (id < 0 || id >= num_blocks)
          return fail(PA_ERR_INVALID, "%s: block_tables[%d][%d] = %d outside [0, %d)", who, s, j,
                      id, num_blocks);
      }
    }
    if (new_k) {
      const pa_status r = check_append_slots(lens, tab, num_seqs, block_size, max_blocks_per_seq, who);
      if (r != PA_OK) return r;
    }
  }

  // the most waves any call with these shapes may use, then what the device holds at once
  const long long t_max = (long long)num_seqs * num_kv_heads * tiles_of(max_seq_len);
  int waves = 0;
  hipError_t e = decode_waves(*dec, &waves);
  if (e != hipSuccess) return hip_fail(e, "pa_decode occupancy query");
  waves = (int)std::min<long long>(waves, std::max<long long>(1, waves_used(t_max, kMaxWaves)));
  if (requested_waves() > 0) waves = std::min(waves, requested_waves());

  p->q = q;
  p->k_cache = k_cache;
  p->v_cache = v_cache;
  p->block_tables = block_tables;
  p->seq_lens = seq_lens;
  p->out = out;
  p->new_k = new_k;
  p->new_v = new_v;
  p->q_start = nullptr;
  p->rows = group;
  p->total_q = 0;
  p->shared = 0;
  p->ws_meta = nullptr;
  p->ws_ml = nullptr;
  p->ws_acc = nullptr;
  p->num_seqs = num_seqs;
  p->num_heads = num_heads;
  p->num_kv_heads = num_kv_heads;
  p->group = group;
  p->head_dim = head_dim;
  p->block_size = block_size;
  p->num_blocks = num_blocks;
  p->max_blocks_per_seq = max_blocks_per_seq;
  p->max_seq_len = max_seq_len;
  p->num_waves = waves;
  p->tail_div = tail_divisor();
  p->tail_pieces = tail_pieces();
  p->scale_log2e = (float)((double)scale * 1.4426950408889634074);
  p->merge_blocks = (waves * (p->tail_pieces + 1) + 3) / 4;
  // one 16-byte piece of a newest K and V row per thread
  const long long pieces = (long long)num_seqs * num_kv_heads * head_dim * (dtype == PA_F32 ? 4 : 2) / 16;
  if (new_k && (pieces + 255) / 256 > (1LL << 30))
    return fail(PA_ERR_UNSUPPORTED, "%s: more than 2^38 bytes of new rows", who);
  p->append_blocks = new_k ? (int)((pieces + 255) / 256) : 0;
  return PA_OK;
}

// Point the parameters at a workspace laid out as `ws` describes, then launch the decode
// kernel and the merge kernel (which also resets the tail counter for the next call).
pa_status launch_decode(DecodeParams* p, const void* dec, const void* red, char* base,
                        const WorkspaceLayout& ws, hipStream_t st) {
  p->ws_meta = reinterpret_cast<int*>(base);
  p->ws_ml = reinterpret_cast<float*>(base + ws.ml_offset);
  p->ws_acc = reinterpret_cast<float*>(base + ws.acc_offset);
  void* kargs[] = {p};
  // four waves per workgroup: one workgroup per CU, one wave per SIMD
  hipError_t e = hipLaunchKernel(dec, dim3((p->num_waves + 3) / 4), dim3(256), kargs, 0, st);
  if (e != hipSuccess) return hip_fail(e, "pa_decode launch");
  e = hipLaunchKernel(red, dim3(p->merge_blocks + p->append_blocks), dim3(256), kargs, 0, st);
  if (e != hipSuccess) return hip_fail(e, "pa_decode merge launch");
  return PA_OK;
}

// Clears the workspace header (the tail counter must start at 0) with a kernel rather
// than hipMemsetAsync, so the set-up is also valid inside a stream capture.
__global__ void clear_header_kernel(int* hdr) { hdr[threadIdx.x] = 0; }

// Device address of `scratch` on the current device, looked up (and its header
// cleared, on `st`) the first time this device is seen.
pa_status scratch_address(hipStream_t st, char** out) {
  static std::mutex mu;
  static std::map<int, char*> by_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "pa_decode_no_alloc: hipGetDevice");
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_device.find(dev);
  if (it != by_device.end()) {
    *out = it->second;
    return PA_OK;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "pa_decode_no_alloc: hipGetSymbolAddress");
  hipLaunchKernelGGL(clear_header_kernel, dim3(1), dim3(64), 0, st, static_cast<int*>(ptr));
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "pa_decode_no_alloc: clearing the workspace header");
  by_device[dev] = static_cast<char*>(ptr);
  *out = static_cast<char*>(ptr);
  return PA_OK;
}

}  // namespace

namespace pagedkv {

size_t multi_query_rows_workspace(int num_seqs, int num_kv_heads, int head_dim, int max_seq_len,
                                  int rows) {
  const long long t_max = (long long)num_seqs * num_kv_heads * tiles_of(max_seq_len);
  return layout_for(waves_used(t_max, kMaxWaves), kMaxTailPieces, rows, head_dim).total;
}

bool multi_query_rows_apply(pa_dtype dtype, int num_seqs, int num_heads, int num_kv_heads,
                            int head_dim, int block_size, int max_q_len, int max_seq_len) {
  const long long rows = (long long)max_q_len * (num_heads / num_kv_heads);
  return dtype != PA_F32 && rows >= 1 && rows <= 16 && (head_dim == 64 || head_dim == 128) &&
         valid_block_size(block_size) && num_seqs <= kLdsSeqs &&
         (long long)num_seqs * tiles_of(max_seq_len) < (1LL << 31) - 1;
}

pa_status multi_query_rows(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* q_start, int num_seqs, int total_q, int num_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_q_len, int max_seq_len, float scale,
                           pa_dtype dtype, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t st) {
  DecodeParams p;
  const void* dec = nullptr;
  const void* red = nullptr;
  bool skip = false;
  pa_status r = prepare_decode(DecodeVariant::kRows, q, k_cache, v_cache, nullptr, nullptr,
                               block_tables, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                               block_size, num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype,
                               out, st, "pa_multi_query", nullptr, 0, false, &p, &dec, &red, &skip);
  if (r != PA_OK || skip) return r;
  p.q_start = q_start;
  p.rows = max_q_len * (num_heads / num_kv_heads);
  p.total_q = total_q;
  p.tail_div = rows_tail_divisor();
  const long long t_max = (long long)num_seqs * num_kv_heads * tiles_of(max_seq_len);
  const WorkspaceLayout ws = layout_for(waves_used(t_max, kMaxWaves), kMaxTailPieces, p.rows, head_dim);
  if (!workspace || workspace_bytes < ws.total)
    return fail(PA_ERR_WORKSPACE, "pa_multi_query: workspace of %zu bytes, %zu needed",
                workspace ? workspace_bytes : (size_t)0, ws.total);
  // The workspace carries no state between pa_multi_query calls.  Without tail parts
  // (the default) nothing reads the counter that hands them out, and the decode kernel
  // writes the chunk count and every chunk record itself; with them the counter is
  // cleared first (a kernel, not a memset, so that a capture stays valid).
  char* base = static_cast<char*>(workspace);
  if (p.tail_div > 0) {
    hipLaunchKernelGGL(clear_header_kernel, dim3(1), dim3(64), 0, st, reinterpret_cast<int*>(base));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pa_multi_query: clearing the workspace header");
  }
  return launch_decode(&p, dec, red, base, ws, st);
}

namespace {

// pa_decode_shared_prefix on the rows mode.  Group j's members are taken in blocks of
// `mpb` (at most 16 / group); block v = j * cpg + c holds members
// group_start[j] + c * mpb ... (none when the group is smaller).  Each block's table is
// laid out as: the group's prefix, cut down to whole units (a unit is max(block size, 16)
// tokens, so every region starts on a tile and on a block), read once; then, for each
// member in order, its tokens past that prefix, padded to whole units.  Member i of the
// block is row i (with its group's heads); the prefix is everyone's.
constexpr long long kSharedTableBytes = 256LL << 20;

struct SharedRowsLayout {
  int mpb = 0;          // members per block
  int cpg = 0;          // blocks per group
  int vgroups = 0;      // blocks of all groups: the "sequences" the decode kernel sees
  int unit = 0;         // region alignment in tokens
  int max_vlen = 0;     // bound on a laid-out length
  int max_vblocks = 0;  // entries per laid-out table
  WorkspaceLayout dec{0, 0, 0, 0};
  size_t table_off = 0, lens_off = 0, qs_off = 0, total = 0;
  bool ok = false;      // the shapes fit the decode kernel's LDS tables and the length bound
};

SharedRowsLayout shared_rows_layout(int num_seqs, int num_groups, int num_heads, int num_kv_heads,
                                    int head_dim, int block_size, int max_group_size, int max_seq_len) {
  SharedRowsLayout L;
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || num_groups <= 0 ||
      max_group_size <= 0 || max_seq_len < 0 || !valid_block_size(block_size))
    return L;
  const int group = num_heads / num_kv_heads;
  if (group > 16) return L;
  L.mpb = std::min(16 / group, max_group_size);
  L.cpg = (max_group_size + L.mpb - 1) / L.mpb;
  const long long vg = (long long)num_groups * L.cpg;
  L.unit = std::max(block_size, kTileTokens);
  const long long per = ((long long)max_seq_len + L.unit - 1) / L.unit * L.unit;
  const long long vlen = std::max<long long>(per * (L.mpb + 1), L.unit);
  // (tables of more than kSharedTableBytes, from long sequences in many large groups, are
  // left to the split kernel rather than held in the workspace)
  if (vg > kLdsSeqs || vlen > kMaxSeqLen || vg * tiles_of((int)vlen) >= (1LL << 31) - 1 ||
      vg * (vlen / block_size) * (long long)sizeof(int32_t) > kSharedTableBytes)
    return L;
  L.vgroups = (int)vg;
  L.max_vlen = (int)vlen;
  L.max_vblocks = L.max_vlen / block_size;
  const long long t_max = (long long)num_seqs * num_kv_heads * tiles_of(max_seq_len);
  L.dec = layout_for(waves_used(t_max, kMaxWaves), kMaxTailPieces, L.mpb * group, head_dim);
  L.table_off = align_up(L.dec.total, 256);
  L.lens_off = L.table_off + align_up((size_t)L.vgroups * L.max_vblocks * sizeof(int32_t), 256);
  L.qs_off = L.lens_off + align_up((size_t)L.vgroups * sizeof(int32_t), 256);
  L.total = L.qs_off + ((size_t)L.vgroups + 1) * sizeof(int32_t);
  L.ok = true;
  return L;
}

struct SharedLayoutArgs {
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* group_start;
  const int32_t* prefix_lens;
  int32_t* vtable;
  int32_t* vlens;
  int32_t* vqs;
  char* out;
  int num_seqs, cpg, mpb, vgroups, block_size, unit;
  int max_blocks_per_seq, max_seq_len, num_blocks, max_vblocks;
  int out_row_bytes;  // one sequence's output rows (all heads)
};

// Workgroup (v, y) writes entries 256 y .. 256 y + 255 of member block v's table;
// workgroup (v, 0) also its length and first member row, and zeros for the output of
// every empty member (which sees no token).  Each workgroup works out the block's regions
// itself, so the table takes three dependent rounds of loads (group bounds, member
// lengths, block ids).  Index data outside the contract is clamped so that every read
// stays in its array.
__global__ __launch_bounds__(256) void shared_layout_kernel(SharedLayoutArgs a) {
  __shared__ int s_len[16], s_start[16], s_tail[16];
  const int v = blockIdx.x;
  const int lane = threadIdx.x;
  const bool first = blockIdx.y == 0;
  const int j = v / a.cpg, c = v - j * a.cpg;
  const int ga = min(max(a.group_start[j], 0), a.num_seqs);
  const int gb = min(max(a.group_start[j + 1], ga), a.num_seqs);
  const int m0 = (int)min((long long)ga + (long long)c * a.mpb, (long long)gb);
  const int nq = min(m0 + a.mpb, gb) - m0;
  const int B = a.block_size, U = a.unit;
  int P = nq > 0 ? min(max(a.prefix_lens[j], 0), a.max_seq_len) : 0;
  P = P / U * U;
  if (lane < nq) s_len[lane] = min(max(a.seq_lens[m0 + lane], 0), a.max_seq_len);
  __syncthreads();
  if (lane == 0) {
    int S = P;
    for (int i = 0; i < nq; ++i) {
      const int t = max(s_len[i] - P, 0);
      s_start[i] = S;
      s_tail[i] = t;
      S += (t + U - 1) / U * U;
    }
    if (first) {
      a.vqs[v] = m0;
      if (v == a.vgroups - 1) a.vqs[a.vgroups] = a.num_seqs;
      a.vlens[v] = nq > 0 ? s_start[nq - 1] + s_tail[nq - 1] : 0;
    }
  }
  __syncthreads();
  const int Lv = nq > 0 ? s_start[nq - 1] + s_tail[nq - 1] : 0;
  const int nvb = (Lv + B - 1) / B;
  for (int k = blockIdx.y * 256 + lane; k < nvb; k += 256 * gridDim.y) {
    const int x = k * B;
    int own = kSharedAll, m = m0, idx = k, e = min(P - x, 32);
    if (x >= P) {
      own = 0;
      for (int i = 0; i < nq; ++i)
        if (x >= s_start[i] && x - s_start[i] < (s_tail[i] + U - 1) / U * U) own = i;
      m = m0 + own;
      const int mb = max((s_len[own] + B - 1) / B, 1);
      idx = min(P / B + (x - s_start[own]) / B, mb - 1);
      e = s_start[own] + s_tail[own] - x;
    }
    e = min(max(e, 1), 32);
    int id = a.block_tables[(size_t)m * a.max_blocks_per_seq + idx];
    id = (unsigned)id < (unsigned)a.num_blocks ? id : 0;
    a.vtable[(size_t)v * a.max_vblocks + k] =
        (int)((unsigned)id | ((unsigned)(e - 1) << kSharedEndShift) | ((unsigned)own << kSharedOwnerShift));
  }
  for (int i = 0; i < nq && first; ++i) {
    if (s_len[i] != 0) continue;
    uint4* o = reinterpret_cast<uint4*>(a.out + (size_t)(m0 + i) * a.out_row_bytes);
    for (int x = lane; x < a.out_row_bytes / 16; x += 256) o[x] = make_uint4(0u, 0u, 0u, 0u);
  }
}

}  // namespace

bool shared_rows_apply(pa_dtype dtype, int num_groups, int num_heads, int num_kv_heads,
                       int head_dim, int block_size, int num_blocks, int max_group_size,
                       int max_seq_len) {
  if (dtype == PA_F32 || (head_dim != 64 && head_dim != 128) || !valid_block_size(block_size) ||
      num_blocks <= 0 || (unsigned)num_blocks > kSharedIdMask + 1u)
    return false;
  return shared_rows_layout(0, num_groups, num_heads, num_kv_heads, head_dim, block_size,
                            max_group_size, max_seq_len).ok;
}

size_t shared_rows_workspace(int num_seqs, int num_groups, int num_heads, int num_kv_heads,
                             int head_dim, int block_size, int max_group_size, int max_seq_len) {
  const SharedRowsLayout L = shared_rows_layout(num_seqs, num_groups, num_heads, num_kv_heads,
                                                head_dim, block_size, max_group_size, max_seq_len);
  return L.ok ? L.total : 0;
}

pa_status shared_rows(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* seq_lens,
                      const int32_t* group_start, const int32_t* prefix_lens, int num_seqs,
                      int num_groups, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int max_blocks_per_seq, int max_group_size,
                      int max_seq_len, float scale, pa_dtype dtype, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t st) {
  const char* who = "pa_decode_shared_prefix";
  const SharedRowsLayout L = shared_rows_layout(num_seqs, num_groups, num_heads, num_kv_heads,
                                                head_dim, block_size, max_group_size, max_seq_len);
  if (!L.ok) return fail(PA_ERR_UNSUPPORTED, "%s: shapes outside the rows path", who);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace))
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed (16-byte aligned)", who,
                workspace ? workspace_bytes : (size_t)0, L.total);
  DecodeParams p;
  const void* dec = nullptr;
  const void* red = nullptr;
  bool skip = false;
  pa_status r = prepare_decode(DecodeVariant::kRows, q, k_cache, v_cache, nullptr, nullptr,
                               block_tables, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                               block_size, num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype,
                               out, st, who, nullptr, 0, false, &p, &dec, &red, &skip);
  if (r != PA_OK || skip) return r;
  char* base = static_cast<char*>(workspace);
  SharedLayoutArgs la;
  la.block_tables = block_tables;
  la.seq_lens = seq_lens;
  la.group_start = group_start;
  la.prefix_lens = prefix_lens;
  la.vtable = reinterpret_cast<int32_t*>(base + L.table_off);
  la.vlens = reinterpret_cast<int32_t*>(base + L.lens_off);
  la.vqs = reinterpret_cast<int32_t*>(base + L.qs_off);
  la.out = static_cast<char*>(out);
  la.num_seqs = num_seqs;
  la.cpg = L.cpg;
  la.mpb = L.mpb;
  la.vgroups = L.vgroups;
  la.block_size = block_size;
  la.unit = L.unit;
  la.max_blocks_per_seq = max_blocks_per_seq;
  la.max_seq_len = max_seq_len;
  la.num_blocks = num_blocks;
  la.max_vblocks = L.max_vblocks;
  la.out_row_bytes = num_heads * head_dim * (dtype == PA_F32 ? 4 : 2);
  const unsigned parts = (unsigned)std::min((L.max_vblocks + 255) / 256, 65535);
  hipLaunchKernelGGL(shared_layout_kernel, dim3((unsigned)L.vgroups, parts), dim3(256), 0, st, la);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "pa_decode_shared_prefix layout launch");
  p.block_tables = la.vtable;
  p.seq_lens = la.vlens;
  p.num_seqs = L.vgroups;
  p.max_blocks_per_seq = L.max_vblocks;
  p.max_seq_len = L.max_vlen;
  p.q_start = la.vqs;
  p.rows = L.mpb * (num_heads / num_kv_heads);
  p.total_q = num_seqs;
  p.shared = 1;
  p.tail_div = rows_tail_divisor();
  if (p.tail_div > 0) {
    hipLaunchKernelGGL(clear_header_kernel, dim3(1), dim3(64), 0, st, reinterpret_cast<int*>(base));
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pa_decode_shared_prefix: clearing the workspace header");
  }
  return launch_decode(&p, dec, red, base, L.dec, st);
}

}  // namespace pagedkv

extern "C" {

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                    int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    int max_blocks_per_seq, int max_seq_len, float scale, pa_dtype dtype, void* out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  DecodeParams p;
  const void* dec = nullptr;
  const void* red = nullptr;
  bool skip = false;
  pa_status r = prepare_decode(DecodeVariant::kStream, q, k_cache, v_cache, nullptr, nullptr,
                               block_tables, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                               block_size, num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype,
                               out, st, "pa_decode", workspace, workspace_bytes, true, &p, &dec, &red,
                               &skip);
  if (r != PA_OK || skip) return r;
  const WorkspaceLayout ws = plan_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len);
  return launch_decode(&p, dec, red, static_cast<char*>(workspace), ws, st);
}

pa_status pa_decode_cached(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                           int num_heads, int num_kv_heads, int head_dim, int block_size,
                           int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                           pa_dtype dtype, void* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  DecodeParams p;
  const void* dec = nullptr;
  const void* red = nullptr;
  bool skip = false;
  pa_status r = prepare_decode(DecodeVariant::kCached, q, k_cache, v_cache, nullptr, nullptr,
                               block_tables, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                               block_size, num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype,
                               out, st, "pa_decode_cached", workspace, workspace_bytes, true, &p,
                               &dec, &red, &skip);
  if (r != PA_OK || skip) return r;
  const WorkspaceLayout ws = plan_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len);
  return launch_decode(&p, dec, red, static_cast<char*>(workspace), ws, st);
}

pa_status pa_decode_append(const void* q, const void* new_k, const void* new_v, void* k_cache,
                           void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                           int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int max_blocks_per_seq, int max_seq_len,
                           float scale, pa_dtype dtype, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  DecodeParams p;
  const void* dec = nullptr;
  const void* red = nullptr;
  bool skip = false;
  if (num_seqs > 0 && (!new_k || !new_v))
    return fail(PA_ERR_INVALID, "pa_decode_append: null pointer argument");
  pa_status r = prepare_decode(DecodeVariant::kAppend, q, k_cache, v_cache, new_k, new_v,
                               block_tables, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                               block_size, num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype,
                               out, st, "pa_decode_append", workspace, workspace_bytes, true, &p, &dec,
                               &red, &skip);
  if (r != PA_OK || skip) return r;
  const WorkspaceLayout ws = plan_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len);
  return launch_decode(&p, dec, red, static_cast<char*>(workspace), ws, st);
}

size_t pa_decode_no_alloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

pa_status pa_decode_no_alloc(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                             int num_heads, int num_kv_heads, int head_dim, int block_size,
                             int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                             pa_dtype dtype, void* out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  DecodeParams p;
  const void* dec = nullptr;
  const void* red = nullptr;
  bool skip = false;
  pa_status r = prepare_decode(DecodeVariant::kStream, q, k_cache, v_cache, nullptr, nullptr,
                               block_tables, seq_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                               block_size, num_blocks, max_blocks_per_seq, max_seq_len, scale, dtype,
                               out, st, "pa_decode_no_alloc", nullptr, 0, false, &p, &dec, &red,
                               &skip);
  if (r != PA_OK || skip) return r;
  // laid out for the waves this launch actually uses and its tail parts
  const WorkspaceLayout ws = layout_for(p.num_waves, p.tail_pieces, p.group, p.head_dim);
  if (ws.total > kNoAllocScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "pa_decode_no_alloc: this call needs %zu bytes of workspace, above the built-in "
                "%zu (%d waves, %d query heads per KV head, head_dim %d); use pa_decode with a "
                "caller-owned workspace", ws.total, kNoAllocScratchBytes, p.num_waves, p.group,
                p.head_dim);
  char* base = nullptr;
  r = scratch_address(st, &base);
  if (r != PA_OK) return r;
  return launch_decode(&p, dec, red, base, ws, st);
}

}  // extern "C"
