// Host-side block manager: the pool of physical blocks, one block table per
// sequence, reference counts, and the slot and copy-on-write decisions a decode
// step needs ("LLM 注意力与计算内核精读笔记 · 05 PagedAttention 与 KV 显存管理",
// §3 and §5 ①②: blocks taken on demand, a new block only when the last one is
// full; §6.1, §6.2 and §12 题4: shared blocks, reference counts, copy before
// writing into a shared block, release when the count reaches zero).
//
// This file holds host code only.  It produces the index inputs of the kernels:
// block tables and lengths for pa_decode, one slot per new token for
// pa_write_kv, and (src, dst) pairs for pa_copy_blocks.
#include <stdint.h>

#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

#include "common.h"
#include "pagedkv.h"

struct pa_block_manager {
  int num_blocks = 0;
  int block_size = 0;
  std::deque<int32_t> free_list;     // taken from the front, released to the back
  std::vector<int32_t> ref;          // sharers of each physical block
  struct Seq {
    std::vector<int32_t> table;      // logical block -> physical block
    int64_t len = 0;                 // tokens written
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
                       pa_block_manager** out) {
  if (!out) return bm_fail(PA_ERR_INVALID, "pa_bm_create: null output pointer");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return bm_fail(PA_ERR_INVALID, "pa_bm_create: num_blocks and block_size must be positive");
  auto* bm = new pa_block_manager;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
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
  for (int32_t b : it->second.table)
    if (--bm->ref[b] == 0) bm->free_list.push_back(b);
  bm->seqs.erase(it);
  return PA_OK;
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
