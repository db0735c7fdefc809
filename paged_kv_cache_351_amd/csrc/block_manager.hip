// Host-side block manager: the pool of physical blocks, one block table per
// sequence, reference counts, and the slot and copy-on-write decisions a decode
// step needs ("LLM 注意力与计算内核精读笔记 · 05 PagedAttention 与 KV 显存管理",
// §3 and §5 ①②: blocks taken on demand, a new block only when the last one is
// full; §5 ③: a preempted request's blocks move to CPU RAM and come back through
// its block table; §6.1, §6.2 and §12 题4: shared blocks, reference counts, copy
// before writing into a shared block, release when the count reaches zero).
//
// This file holds host code only.  It produces the index inputs of the kernels:
// block tables and lengths for pa_decode, one slot per new token for
// pa_write_kv, and (src, dst) pairs for pa_copy_blocks and pa_swap_blocks.
#include <stdint.h>

#include <deque>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "common.h"
#include "pagedkv.h"

struct pa_block_manager {
  int num_blocks = 0;
  int block_size = 0;
  std::deque<int32_t> free_list;     // taken from the front, released to the back
  std::vector<int32_t> ref;          // sharers of each physical block
  int num_cpu_blocks = 0;            // host pool of swapped-out blocks
  std::deque<int32_t> cpu_free;
  std::vector<int32_t> cpu_ref;
  struct Seq {
    std::vector<int32_t> table;      // logical block -> block of the pool it lives in
    int64_t len = 0;                 // tokens written
    bool swapped = false;            // table names host blocks
  };
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }
};

namespace {

pa_status bm_fail(pa_status st, const char* what) {
  pagedkv::set_last_error(what);
  return st;
}

}  // namespace

extern "C" {

pa_status pa_bm_create(int num_blocks, int block_size, const int32_t* free_order,
                       int num_cpu_blocks, pa_block_manager** out) {
  if (!out) return bm_fail(PA_ERR_INVALID, "pa_bm_create: null output pointer");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || num_cpu_blocks < 0)
    return bm_fail(PA_ERR_INVALID, "pa_bm_create: num_blocks and block_size must be positive, "
                   "num_cpu_blocks not negative");
  auto* bm = new pa_block_manager;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->num_cpu_blocks = num_cpu_blocks;
  bm->cpu_ref.assign(num_cpu_blocks, 0);
  for (int32_t b = 0; b < num_cpu_blocks; ++b) bm->cpu_free.push_back(b);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return bm_fail(PA_ERR_INVALID, "pa_bm_create: free_order is not a permutation of 0..num_blocks-1");
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq, int64_t num_tokens) {
  if (!bm) return bm_fail(PA_ERR_INVALID, "pa_bm_allocate: null manager");
  if (num_tokens < 0) return bm_fail(PA_ERR_INVALID, "pa_bm_allocate: negative token count");
  if (bm->seqs.count(seq)) return bm_fail(PA_ERR_INVALID, "pa_bm_allocate: sequence already allocated");
  const int64_t n = (num_tokens + bm->block_size - 1) / bm->block_size;
  if ((int64_t)bm->free_list.size() < n)
    return bm_fail(PA_ERR_NO_BLOCKS, "pa_bm_allocate: not enough free blocks");
  pa_block_manager::Seq s;
  s.table.reserve(n);
  for (int64_t i = 0; i < n; ++i) s.table.push_back(bm->take());
  s.len = num_tokens;
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status pa_bm_append_slot(pa_block_manager* bm, int64_t seq, int64_t* slot, int32_t* cow_src,
                            int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst)
    return bm_fail(PA_ERR_INVALID, "pa_bm_append_slot: null argument");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return bm_fail(PA_ERR_INVALID, "pa_bm_append_slot: unknown sequence");
  if (it->second.swapped) return bm_fail(PA_ERR_INVALID, "pa_bm_append_slot: sequence is swapped out");
  auto& s = it->second;
  const int B = bm->block_size;
  const int64_t pos = s.len;
  const size_t lb = (size_t)(pos / B);
  *cow_src = -1;
  *cow_dst = -1;
  if (lb == s.table.size()) {  // last block full (or none): take a new one
    if (bm->free_list.empty()) return bm_fail(PA_ERR_NO_BLOCKS, "pa_bm_append_slot: no free block");
    s.table.push_back(bm->take());
  } else {
    const int32_t last = s.table[lb];
    if (bm->ref[last] > 1) {  // still shared: copy it before writing
      if (bm->free_list.empty()) return bm_fail(PA_ERR_NO_BLOCKS, "pa_bm_append_slot: no free block");
      const int32_t fresh = bm->take();
      bm->ref[last] -= 1;
      s.table[lb] = fresh;
      *cow_src = last;
      *cow_dst = fresh;
    }
  }
  s.len = pos + 1;
  *slot = (int64_t)s.table[lb] * B + pos % B;
  return PA_OK;
}

pa_status pa_bm_append_step(pa_block_manager* bm, const int64_t* seqs, int num_seqs,
                            int32_t* slot_mapping, int32_t* pairs, int* num_pairs) {
  if (!bm || num_seqs < 0 || !num_pairs) return bm_fail(PA_ERR_INVALID, "pa_bm_append_step: bad arguments");
  if (num_seqs > 0 && (!seqs || !slot_mapping || !pairs))
    return bm_fail(PA_ERR_INVALID, "pa_bm_append_step: null array");
  if ((int64_t)bm->num_blocks * bm->block_size > INT32_MAX)
    return bm_fail(PA_ERR_UNSUPPORTED, "pa_bm_append_step: pool has more than 2^31 slots");
  // Dry run: every sequence must exist once, and the blocks the step takes --
  // one per full last block, one per write into a block that is still shared
  // when its turn comes -- must all be free, so that a failure changes nothing.
  std::unordered_map<int64_t, char> once;
  std::unordered_map<int32_t, int32_t> gone;  // sharers that left a block earlier in the step
  int64_t need = 0;
  for (int i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return bm_fail(PA_ERR_INVALID, "pa_bm_append_step: unknown sequence");
    if (!once.emplace(seqs[i], 1).second)
      return bm_fail(PA_ERR_INVALID, "pa_bm_append_step: a sequence is listed twice");
    if (it->second.swapped) return bm_fail(PA_ERR_INVALID, "pa_bm_append_step: a sequence is swapped out");
    const auto& sq = it->second;
    const size_t lb = (size_t)(sq.len / bm->block_size);
    if (lb == sq.table.size()) {
      ++need;
    } else {
      const int32_t last = sq.table[lb];
      if (bm->ref[last] - gone[last] > 1) {
        ++need;
        ++gone[last];
      }
    }
  }
  if (need > (int64_t)bm->free_list.size())
    return bm_fail(PA_ERR_NO_BLOCKS, "pa_bm_append_step: not enough free blocks for the step");
  int np = 0;
  for (int i = 0; i < num_seqs; ++i) {
    int64_t slot;
    int32_t src, dst;
    const pa_status st = pa_bm_append_slot(bm, seqs[i], &slot, &src, &dst);
    if (st != PA_OK) return st;  // unreachable after the dry run
    slot_mapping[i] = (int32_t)slot;
    if (src >= 0) {
      pairs[2 * np] = src;
      pairs[2 * np + 1] = dst;
      ++np;
    }
  }
  *num_pairs = np;
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return bm_fail(PA_ERR_INVALID, "pa_bm_fork: null manager");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return bm_fail(PA_ERR_INVALID, "pa_bm_fork: unknown parent");
  if (it->second.swapped) return bm_fail(PA_ERR_INVALID, "pa_bm_fork: parent is swapped out");
  if (bm->seqs.count(child)) return bm_fail(PA_ERR_INVALID, "pa_bm_fork: child already exists");
  pa_block_manager::Seq c = it->second;
  for (int32_t b : c.table) bm->ref[b] += 1;
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status pa_bm_free(pa_block_manager* bm, int64_t seq) {
  if (!bm) return bm_fail(PA_ERR_INVALID, "pa_bm_free: null manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return bm_fail(PA_ERR_INVALID, "pa_bm_free: unknown sequence");
  auto& ref = it->second.swapped ? bm->cpu_ref : bm->ref;
  auto& free_list = it->second.swapped ? bm->cpu_free : bm->free_list;
  for (int32_t b : it->second.table)
    if (--ref[b] == 0) free_list.push_back(b);
  bm->seqs.erase(it);
  return PA_OK;
}

namespace {

// Move the listed sequences' blocks to the other pool.  Each distinct block
// they reference moves once, in first-reference order, to the next free block
// of the target pool, carrying the number of listed sharers as its count; the
// source block loses those sharers and is released at zero.  All or nothing.
pa_status bm_move(pa_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* pairs,
                  int pairs_cap, int* num_pairs, bool to_cpu, const char* who) {
  static thread_local std::string msg;
  auto failf = [&](pa_status st, const char* what) {
    msg = std::string(who) + ": " + what;
    return bm_fail(st, msg.c_str());
  };
  if (!bm || num_seqs < 0 || !num_pairs || pairs_cap < 0) return failf(PA_ERR_INVALID, "bad arguments");
  if (num_seqs > 0 && !seqs) return failf(PA_ERR_INVALID, "null array");
  std::unordered_map<int64_t, char> once;
  std::vector<std::pair<int32_t, int32_t>> moving;  // (source block, leaving sharers)
  std::unordered_map<int32_t, size_t> where;
  for (int i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return failf(PA_ERR_INVALID, "unknown sequence");
    if (!once.emplace(seqs[i], 1).second) return failf(PA_ERR_INVALID, "a sequence is listed twice");
    if (it->second.swapped == to_cpu)
      return failf(PA_ERR_INVALID, to_cpu ? "sequence already swapped out" : "sequence is not swapped out");
    for (int32_t b : it->second.table) {
      auto w = where.find(b);
      if (w == where.end()) {
        where.emplace(b, moving.size());
        moving.emplace_back(b, 1);
      } else {
        moving[w->second].second += 1;
      }
    }
  }
  auto& src_ref = to_cpu ? bm->ref : bm->cpu_ref;
  auto& src_free = to_cpu ? bm->free_list : bm->cpu_free;
  auto& dst_ref = to_cpu ? bm->cpu_ref : bm->ref;
  auto& dst_free = to_cpu ? bm->cpu_free : bm->free_list;
  if (moving.size() > dst_free.size())
    return failf(PA_ERR_NO_BLOCKS, to_cpu ? "not enough free host blocks" : "not enough free blocks");
  if ((int64_t)moving.size() > pairs_cap) return failf(PA_ERR_INVALID, "pairs array too small");
  if (!moving.empty() && !pairs) return failf(PA_ERR_INVALID, "null pairs array");
  std::unordered_map<int32_t, int32_t> new_id;
  for (size_t i = 0; i < moving.size(); ++i) {
    const int32_t d = dst_free.front();
    dst_free.pop_front();
    dst_ref[d] = moving[i].second;
    new_id.emplace(moving[i].first, d);
    pairs[2 * i] = moving[i].first;
    pairs[2 * i + 1] = d;
  }
  for (const auto& m : moving)
    if ((src_ref[m.first] -= m.second) == 0) src_free.push_back(m.first);
  for (int i = 0; i < num_seqs; ++i) {
    auto& sq = bm->seqs[seqs[i]];
    for (int32_t& b : sq.table) b = new_id[b];
    sq.swapped = to_cpu;
  }
  *num_pairs = (int)moving.size();
  return PA_OK;
}

}  // namespace

pa_status pa_bm_swap_out(pa_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* pairs,
                         int pairs_cap, int* num_pairs) {
  return bm_move(bm, seqs, num_seqs, pairs, pairs_cap, num_pairs, true, "pa_bm_swap_out");
}

pa_status pa_bm_swap_in(pa_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* pairs,
                        int pairs_cap, int* num_pairs) {
  return bm_move(bm, seqs, num_seqs, pairs, pairs_cap, num_pairs, false, "pa_bm_swap_in");
}

int pa_bm_num_free_cpu(const pa_block_manager* bm) { return bm ? (int)bm->cpu_free.size() : -1; }

int pa_bm_cpu_ref_count(const pa_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_cpu_blocks) return -1;
  return bm->cpu_ref[block];
}

int pa_bm_is_swapped(const pa_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

int pa_bm_num_free(const pa_block_manager* bm) { return bm ? (int)bm->free_list.size() : -1; }

int64_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int pa_bm_table(const pa_block_manager* bm, int64_t seq, int32_t* out, int cap) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -1;
  const auto& t = it->second.table;
  if (!out) cap = 0;
  for (int i = 0; i < cap && i < (int)t.size(); ++i) out[i] = t[i];
  return (int)t.size();
}

int pa_bm_ref_count(const pa_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

pa_status pa_bm_batch(const pa_block_manager* bm, const int64_t* seqs, int num_seqs,
                      int32_t* block_tables, int max_blocks_per_seq, int32_t* seq_lens) {
  if (!bm || num_seqs < 0 || max_blocks_per_seq <= 0)
    return bm_fail(PA_ERR_INVALID, "pa_bm_batch: bad arguments");
  if (num_seqs > 0 && (!seqs || !block_tables || !seq_lens))
    return bm_fail(PA_ERR_INVALID, "pa_bm_batch: null array");
  for (int i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return bm_fail(PA_ERR_INVALID, "pa_bm_batch: unknown sequence");
    if (it->second.swapped) return bm_fail(PA_ERR_INVALID, "pa_bm_batch: a sequence is swapped out");
    const auto& t = it->second.table;
    if ((int)t.size() > max_blocks_per_seq)
      return bm_fail(PA_ERR_INVALID, "pa_bm_batch: a table is longer than max_blocks_per_seq");
    if (it->second.len > INT32_MAX) return bm_fail(PA_ERR_INVALID, "pa_bm_batch: length above 2^31");
    int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
    for (int j = 0; j < max_blocks_per_seq; ++j) row[j] = j < (int)t.size() ? t[j] : -1;
    seq_lens[i] = (int32_t)it->second.len;
  }
  return PA_OK;
}

}  // extern "C"
