// pa_multi_query and pa_decode_shared_prefix: validation, launch plans and
// dispatch of the kernels in multi_query.hip.
#include <vector>

#include <algorithm>

#include "decode_params.h"
#include "host_util.h"
#include "multi_query.h"
#include "pagedkv.h"

using namespace pagedkv;

// The entry points keep the C linkage of their declarations in pagedkv.h.

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
  // the sequences are taken longest first (their lengths set most of the items' work),
  // so the last items to start are the shortest
  if (num_seqs > 0)
    pl.order_bytes = ((size_t)num_seqs * sizeof(int32_t) + 255) / 256 * 256;
  if (pl.parts > 1) {
    const size_t slots = (size_t)total_q * num_heads * pl.parts;
    pl.ml_bytes = (slots * 2 * sizeof(float) + 255) / 256 * 256;
    pl.total = pl.ml_bytes + slots * head_dim * sizeof(float);
  }
  pl.total += pl.order_bytes;
  return pl;
}

// PA_MULTI_QUERY_ROWS=0 keeps pa_multi_query on its own kernels for every shape (for
// comparisons); the rows mode is on by default.
bool multi_query_rows_enabled() {
  static const bool v = env_flag("PA_MULTI_QUERY_ROWS", true);
  return v;
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
  // query block whenever it applies, like the other); where the rows mode may apply
  // (16-bit types, at most 16 rows per pair), it covers that mode's too
  size_t n = mq_plan(num_seqs, total_q, num_heads, num_kv_heads, head_dim, max_q_len, max_seq_len, PA_BF16).total;
  const long long rows = (long long)max_q_len * (num_heads / num_kv_heads);
  if (rows >= 1 && rows <= 16 && (head_dim == 64 || head_dim == 128))
    n = std::max(n, multi_query_rows_workspace(num_seqs, num_kv_heads, head_dim, max_seq_len, (int)rows));
  return n;
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
  {
    // the shared-tile kernels address a cache block with 32-bit block and 24-bit row offsets
    const long long row = (long long)num_kv_heads * head_dim * (dtype == PA_F32 ? 4 : 2);
    if (row >= (1LL << 24) || row * block_size >= (1LL << 32))
      return fail(PA_ERR_UNSUPPORTED, "pa_multi_query: %lld bytes per cache slot and %lld per block "
                  "(at most 2^24 - 1 and 2^32 - 1)", row, row * block_size);
  }
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !q_start || !out)
    return fail(PA_ERR_INVALID, "pa_multi_query: null pointer argument");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PA_ERR_INVALID, "pa_multi_query: q, caches and out must be 16-byte aligned");
  const MQPlan pl = mq_plan(num_seqs, total_q, num_heads, num_kv_heads, head_dim, max_q_len, max_seq_len,
                            (int)dtype);
  // the kernel deals (sequence, KV head) units to the 8 XCDs in turn: a multiple of 8
  // units times the items of a unit
  const long long units = (long long)num_seqs * num_kv_heads;
  const long long wgs = (units + 7) / 8 * 8 * ((long long)pl.qblocks * pl.parts);
  if (wgs >= (1LL << 31))
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
  // At most 16 rows per (sequence, KV head) pair (verification of a few drafted tokens):
  // the decode kernels, whose even split of the step over the waves streams the cache
  // faster than one work item per workgroup
  if (multi_query_rows_enabled() &&
      multi_query_rows_apply(dtype, num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_q_len,
                             max_seq_len))
    return multi_query_rows(q, k_cache, v_cache, block_tables, seq_lens, q_start, num_seqs, total_q,
                            num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                            max_blocks_per_seq, max_q_len, max_seq_len, scale, dtype, out, workspace,
                            workspace_bytes, st);
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
  mp.log2_block_size = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  mp.num_blocks = num_blocks;
  mp.max_blocks_per_seq = max_blocks_per_seq;
  mp.max_q_len = max_q_len;
  mp.max_seq_len = max_seq_len;
  mp.tq = pl.tq;
  mp.qblocks = pl.qblocks;
  mp.parts = pl.parts;
  mp.items = pl.items;
  mp.scale_log2e = (float)((double)scale * 1.4426950408889634074);
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
  // the larger of the split kernel's plan and the rows path's (whose tables are largest
  // for 8-token blocks), so that either path fits
  const size_t split = sp_plan(num_seqs, num_groups, num_heads, num_kv_heads, head_dim, max_group_size,
                               max_seq_len).total;
  const size_t rows = shared_rows_workspace(num_seqs, num_groups, num_heads, num_kv_heads, head_dim, 8,
                                            max_group_size, max_seq_len);
  return split > rows ? split : rows;
}

// PA_SHARED_PREFIX_ROWS=0 keeps pa_decode_shared_prefix on the split multi-query kernel
// (for comparisons); read at every call.
static bool shared_prefix_rows_enabled() { return env_flag("PA_SHARED_PREFIX_ROWS", true); }

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
  // (group, KV head) units dealt to the 8 XCDs in turn, as for pa_multi_query
  const long long wgs = ((long long)num_groups * num_kv_heads + 7) / 8 * 8 * ((long long)pl.qblocks * pl.parts);
  if (wgs >= (1LL << 31))
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
  // The decode kernels' rows mode: the step split evenly over one wave per SIMD (the
  // split kernel runs one work item per workgroup and pays a start per item).
  if (shared_prefix_rows_enabled() &&
      shared_rows_apply(dtype, num_groups, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_group_size, max_seq_len) &&
      workspace && aligned16(workspace) &&
      workspace_bytes >= shared_rows_workspace(num_seqs, num_groups, num_heads, num_kv_heads, head_dim,
                                               block_size, max_group_size, max_seq_len))
    return shared_rows(q, k_cache, v_cache, block_tables, seq_lens, group_start, prefix_lens, num_seqs,
                       num_groups, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_group_size, max_seq_len, scale, dtype, out, workspace,
                       workspace_bytes, st);
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
  mp.log2_block_size = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  mp.num_blocks = num_blocks;
  mp.max_blocks_per_seq = max_blocks_per_seq;
  mp.max_q_len = max_group_size;
  mp.max_seq_len = max_seq_len;
  mp.tq = pl.tq;
  mp.qblocks = pl.qblocks;
  mp.parts = pl.parts;
  mp.items = pl.items;
  mp.scale_log2e = (float)((double)scale * 1.4426950408889634074);
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
