/*
 * pagedkv.h -- C ABI of libpagedkv, paged decode attention for MI355X (gfx950).
 *
 * The operations follow three web pages on PagedAttention, cited as
 *   [PA-notes]     "LLM 注意力与计算内核精读笔记 · 05 PagedAttention 与 KV 显存管理"
 *   [vLLM-what]    "vLLM 是什么 PagedAttention 解决了什么"
 *   [PA-explainer] "PagedAttention：分页注意力——推理引擎的显存革命"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer to contiguous row-major
 *   memory owned by the caller.  The library allocates no device memory and
 *   keeps no pointer after a call returns.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Calls only enqueue work and return; results are ready when the
 *   stream reaches that point.  Work issued on one stream runs in order, so
 *   write -> copy -> decode on one stream needs no extra synchronisation.
 * Element types.  pa_dtype names the storage type of q, K/V, new tokens and
 *   the output.  Arithmetic is float32 inside the kernels.
 * Cache pool layout (both K and V, identical):
 *     cache[num_blocks][block_size][num_kv_heads][head_dim]
 *   Each physical block holds block_size consecutive tokens of one sequence
 *   ([PA-notes] §3; per-block [block_size, heads, head_dim] as in
 *   [PA-explainer] "Block结构", with KV heads under GQA as in [vLLM-what]
 *   "1）KV cache 显存估算").  Token t of a sequence is in its logical block
 *   t / block_size at offset t % block_size.
 * Slots.  slot = physical_block * block_size + offset, a flat token index
 *   into the pool.
 * Errors.  Problems the host can see (null pointers, unsupported sizes,
 *   inconsistent dimensions, a workspace too small) return a non-PA_OK status
 *   before anything is enqueued; pa_last_error() then describes it.  Index
 *   data that lives on the device (block tables, slots, pairs) is the
 *   caller's contract and is not checked on the hot path: out-of-range ids
 *   are clamped (decode) or skipped (write, copy) so that no access leaves the
 *   pool, and the result for such entries is unspecified.  Setting the
 *   environment variable PA_DEBUG_CHECK=1 makes every call copy its index
 *   arrays to the host, synchronously, and reject contract violations with
 *   PA_ERR_INVALID before launching.  A failed launch returns PA_ERR_HIP.
 * Thread safety.  Calls may come from any host thread; pa_last_error() is per
 *   thread.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_F32 = 0,  /* float32 */
  PA_F16 = 1,  /* IEEE binary16 */
  PA_BF16 = 2  /* bfloat16 */
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = 1,     /* bad argument or (debug mode) bad index data */
  PA_ERR_UNSUPPORTED = 2, /* valid request outside the compiled kernel set */
  PA_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  PA_ERR_HIP = 4,         /* the HIP runtime reported an error */
  PA_ERR_NO_BLOCKS = 5    /* block manager: the pool has no free block left */
} pa_status;

/* Library ABI version (incremented on any signature change or new entry point). */
int pa_version(void);

/* Message for the last non-PA_OK status returned on the calling thread
 * ("" if none).  The string stays valid until the next call on that thread. */
const char* pa_last_error(void);

/* Bytes of workspace pa_decode needs for these arguments (0 for invalid
 * arguments).  It depends only on the shapes: the number of waves a call may
 * launch is bounded by num_seqs * num_kv_heads * ceil(max_seq_len / 16) / 8
 * and by 2048; each wave's work is cut into at most five chunks, and each chunk
 * needs 16 bytes of bookkeeping plus two partial results of (head_dim + 2)
 * floats per query head of its group, after a 256-byte header. */
size_t pa_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                int max_seq_len);

/*
 * pa_decode -- one decode step of paged attention.
 *
 * For every sequence s and query head h (KV head kv = h / (num_heads /
 * num_kv_heads)), with L = seq_lens[s] tokens:
 *     out[s][h] = sum_t softmax_t(scale * q[s][h] . K_s[t][kv]) * V_s[t][kv]
 * where K_s[t] is read from physical block block_tables[s][t / block_size] at
 * offset t % block_size.  The softmax is normalised over all L tokens of the
 * sequence, across blocks, by merging a running maximum and running sum block
 * by block ([PA-notes] §4; the dense formula with 1/sqrt(d) is [vLLM-what]
 * "2）PagedAttention 算子").  A sequence with L = 0 yields zeros.
 *
 * Work split: the step's (sequence, KV head) pairs are cut into 16-token tiles
 * and the launched waves (as many as the device holds at once) take equal runs
 * of consecutive tiles, whatever the length mix; the last sixteenth of every
 * run (up to an eighth when runs are short, so that a part keeps at least 16
 * tiles) is handed to whichever wave is free first.  A pair cut by a run
 * boundary is finished by a second kernel on the same stream, which merges the
 * pieces' running maxima, sums and accumulators with the same rule.  The boundaries
 * depend only on the lengths, so which wave did which part never changes the
 * result.
 *
 *   q            [num_seqs][num_heads][head_dim]            dtype
 *   k_cache      [num_blocks][block_size][num_kv_heads][head_dim]  dtype
 *   v_cache      same shape as k_cache
 *   block_tables [num_seqs][max_blocks_per_seq] int32: physical block ids;
 *                entries at and past ceil(L / block_size) are never read
 *   seq_lens     [num_seqs] int32, 0 <= L <= max_seq_len
 *   out          [num_seqs][num_heads][head_dim] dtype; must not alias inputs
 *   workspace    device scratch of at least pa_decode_workspace_size(...)
 *                bytes, 256-byte aligned, zero-filled before its first use.
 *                A call leaves it ready for the next one (the counter it
 *                uses to hand out work is back at 0), so it is zeroed once,
 *                not per call.  A first call on a workspace that was not
 *                zeroed may give wrong results but keeps every access inside
 *                the arrays, and still leaves the workspace ready.  Calls
 *                that share a workspace must not run concurrently (put them
 *                on one stream).
 *   max_seq_len  caller's upper bound on every seq_lens[s]; must be
 *                <= max_blocks_per_seq * block_size and <= 2^24.  Lengths
 *                above it are clamped to it, negative lengths to 0.
 * Supported: head_dim in {64, 128}; block_size in {8, 16, 32}; num_heads a
 * multiple of num_kv_heads with group size num_heads / num_kv_heads <= 16.
 * Accumulation is float32; the output is rounded once, to nearest even.  For
 * fp16 and bf16 with 3 or more query heads per KV head, P.V runs on the matrix
 * cores with the softmax weights in the storage type (two bf16 terms, about 16
 * significant bits, or one fp16 term).
 * Results are deterministic on a given device: the same inputs give the same
 * bits (the split depends on the lengths and the device's wave capacity).
 * The current HIP device must be the stream's device.
 */
pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                    int block_size, int num_blocks, int max_blocks_per_seq,
                    int max_seq_len, float scale, pa_dtype dtype, void* out,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_cached -- pa_decode for batches whose sequences share blocks.
 *
 * Same arguments, result (bit for bit), errors and workspace as pa_decode; only
 * the cache policy of the K/V loads differs.  pa_decode reads K/V with the
 * non-temporal hint, since each row is read once per call: the streamed lines
 * do not take room in L2 and the Infinity Cache, which makes it faster when
 * sequences share no blocks.  When sequences of the batch share blocks
 * (parallel samples or beams of one prompt reading its blocks, [PA-notes] §6.1
 * and §6.2), those rows are read once per sequence and the default policy lets
 * the repeated reads hit in the caches: use this call, or
 * pa_decode_shared_prefix, which reads a group's shared blocks once.
 */
pa_status pa_decode_cached(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int max_blocks_per_seq,
                           int max_seq_len, float scale, pa_dtype dtype, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_no_alloc -- pa_decode for callers that cannot allocate device memory
 * (code recorded into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, result and errors as pa_decode, without the
 * workspace: the call uses a workspace built into the library, one array of
 * PA_DECODE_NO_ALLOC_SCRATCH_BYTES bytes of device memory per GPU, which that GPU
 * holds from the first call on it until the process ends.  The call allocates and
 * frees nothing.  The first call on a device looks the array up and clears its
 * header on `stream` (make that first call outside a stream capture); later calls
 * reuse it as a caller-owned workspace is reused.  Every call on one GPU shares
 * that GPU's array, so calls that may overlap on one GPU (different streams,
 * different threads) race and give wrong results: serialise them, e.g. on one
 * stream.  The array holds the workspace of every shape pa_decode supports with
 * the default work split on an MI355X (at most 1,024 waves, two chunks each); a
 * call that would need more (a device with more compute units, or the tuning
 * overrides of the split) returns PA_ERR_WORKSPACE before enqueuing anything.
 * Results are bit-identical to pa_decode's for the same inputs on the same device.
 */
#define PA_DECODE_NO_ALLOC_SCRATCH_BYTES ((size_t)34 << 20)
size_t pa_decode_no_alloc_scratch_bytes(void); /* = PA_DECODE_NO_ALLOC_SCRATCH_BYTES */
pa_status pa_decode_no_alloc(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens,
                             int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int block_size, int num_blocks, int max_blocks_per_seq,
                             int max_seq_len, float scale, pa_dtype dtype, void* out,
                             void* stream);

/*
 * pa_write_kv -- store new tokens' K and V rows into their slots.
 *
 * For every i with 0 <= slot_mapping[i] < num_blocks * block_size:
 *     k_cache[slot / block_size][slot % block_size] = k[i]   (all KV heads)
 *     v_cache[slot / block_size][slot % block_size] = v[i]
 * A negative slot marks a padding token and writes nothing.  This is the
 * append step of on-demand allocation: a new token goes to the next free slot
 * of its sequence's last block, and the host takes a new block only when that
 * one is full ([PA-notes] §5 ②).  The copy is bit-exact.
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim] dtype; must not alias
 *                 the caches
 *   slot_mapping  [num_tokens] int32; two tokens must not name the same slot
 *   k_cache, v_cache  pool layout above
 */
pa_status pa_write_kv(const void* k, const void* v, const int32_t* slot_mapping,
                      void* k_cache, void* v_cache, int num_tokens,
                      int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_decode_append -- the append and the decode of one step in one call: each
 * sequence's newest token (position L - 1, already counted in seq_lens) is stored
 * into its slot, and then every sequence is decoded as by pa_decode.
 *
 * Results are bit-identical to pa_write_kv(new_k, new_v, slots) followed by
 * pa_decode with the same arguments, where slots[s] is the slot the block table
 * assigns to position L - 1 of sequence s: block_tables[s][(L-1) / block_size]
 * * block_size + (L-1) % block_size ([PA-notes] §5 ②: the new token goes to the
 * next free slot of the sequence's last block; the decode itself is [PA-notes]
 * §4).  Sequences with L = 0 append nothing.  The decode kernel reads that
 * token from new_k/new_v instead of the slot, and the merge kernel that follows
 * it on the stream stores the rows into the slot, so the step needs no write
 * launch of its own and no ordering between the write and the decode's reads.
 *
 *   new_k, new_v  [num_seqs][num_kv_heads][head_dim] dtype, 16-byte aligned;
 *                 must not alias the caches
 *   k_cache, v_cache  written at each sequence's newest slot, read elsewhere
 *   other arguments, errors and workspace as for pa_decode
 * Each newest slot must belong to its sequence alone: no two sequences may
 * append into one slot, and no other (sequence, position) of the batch may read
 * it (the copy-on-write contract: a shared last block is copied first).  With
 * PA_DEBUG_CHECK=1 a violation returns PA_ERR_INVALID before anything is
 * enqueued.  Without it the result is undefined but every access stays inside
 * the arrays; a table entry outside [0, num_blocks) at position L - 1 writes
 * nothing.
 */
pa_status pa_decode_append(const void* q, const void* new_k, const void* new_v,
                           void* k_cache, void* v_cache, const int32_t* block_tables,
                           const int32_t* seq_lens, int num_seqs, int num_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, int max_seq_len, float scale,
                           pa_dtype dtype, void* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * pa_copy_blocks -- copy-on-write block duplication.
 *
 * For every pair (src, dst) = (src_dst_pairs[2i], src_dst_pairs[2i+1]):
 *     k_cache[dst] = k_cache[src];  v_cache[dst] = v_cache[src]
 * copying the whole block (every slot and KV head).  Before a sequence writes
 * into a physical block that other sequences still share, the host picks a
 * fresh block, repoints the writer's table entry and asks for this copy
 * ([PA-notes] §6.1 and §12 题4).  All pairs act at once: no dst may be a src
 * of any pair, and no dst may repeat.  Pairs naming ids outside
 * [0, num_blocks) are skipped.  The copy is bit-exact.
 *
 *   src_dst_pairs  [num_pairs][2] int32, device memory
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst_pairs,
                         int num_pairs, int block_size, int num_kv_heads,
                         int head_dim, int num_blocks, pa_dtype dtype, void* stream);

/*
 * Multi-query paged attention -- several query tokens per sequence, causal:
 * the attention of chunked prefill (a long prompt processed in pieces) and of
 * speculative verification (several drafted tokens scored at once), which
 * [PA-explainer] "2026年最新进展" pairs with PagedAttention.
 *
 * Sequence s owns query rows q_start[s] .. q_start[s+1]-1 of q: its last
 * n_s = q_start[s+1] - q_start[s] tokens, whose K/V are already in the cache
 * (pa_write_kv).  seq_lens[s] = L_s counts every cached token including those.
 * Query i of the sequence sits at position p = L_s - n_s + i and attends to
 * tokens 0..p ([PA-notes] §4 blockwise softmax over the sequence's blocks):
 *     out[q_start[s] + i, h] = softmax_{t <= p}(scale * q[.., h] . K_s[t]) V_s[t]
 * with GQA as in pa_decode.  One query per sequence is exactly pa_decode.
 *
 *   q, out         [total_q][num_heads][head_dim], dtype
 *   k_cache, ...   as for pa_decode (block_size any positive value here)
 *   q_start        device int32 [num_seqs + 1], non-decreasing, q_start[0] = 0,
 *                  q_start[num_seqs] = total_q
 *   seq_lens       device int32 [num_seqs], n_s <= L_s <= max_seq_len
 *   max_q_len      host bound on every n_s (no device sync is made)
 *   workspace      pa_multi_query_workspace_size(...) bytes, 16-byte aligned:
 *                  the work plan and partial results; no zero-fill needed (the
 *                  call clears what it counts on)
 *
 * With at most 16 (query, head) rows per (sequence, KV head) (max_q_len *
 * num_heads / num_kv_heads <= 16: verification of a few drafted tokens), fp16
 * or bf16, and block_size 8, 16 or 32, the call runs on the decode kernels:
 * each pair's rows take the 16 columns of the decode's score tile, each row
 * with its own causal limit, and the step is split evenly over the waves as
 * for pa_decode (a clear of the workspace header, the decode kernel, the
 * merge kernel).  Otherwise work is cut into (sequence, KV head, block of query
 * rows, context partition) items; with few items the context is split into
 * partitions that a second kernel merges, in a fixed order.  Head_dim 64 or 128; at most 64
 * query heads per KV head; a cache slot (num_kv_heads * head_dim elements)
 * below 2^24 bytes and a block below 2^32 bytes (PA_ERR_UNSUPPORTED beyond
 * these).  Errors as for pa_decode; index data violating the contract above
 * is clamped so that no access leaves the arrays, with unspecified results
 * (PA_DEBUG_CHECK=1 rejects it).  Results are deterministic.
 */
size_t pa_multi_query_workspace_size(int num_seqs, int total_q, int num_heads, int num_kv_heads,
                                     int head_dim, int max_q_len, int max_seq_len);
pa_status pa_multi_query(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* q_start, int num_seqs, int total_q, int num_heads,
                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                         int max_blocks_per_seq, int max_q_len, int max_seq_len, float scale,
                         pa_dtype dtype, void* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Shared-prefix decode -- pa_decode's result, reading each shared prefix once.
 * Parallel samples of one prompt (and beam candidates) point at the same
 * physical blocks for the prompt ([PA-notes] §6.1, §6.2; [vLLM-what] "3）Prefix
 * Caching"); pa_decode reads those blocks once per sample, this call once per
 * group.  Sequences are listed group by group: group j is sequences
 * group_start[j] .. group_start[j+1]-1, and the first prefix_lens[j] tokens of
 * every member sit in the same physical blocks (the first
 * ceil(prefix_lens[j] / block_size) table entries of all members are equal).
 * Every member's remaining tokens are its own.  The output equals pa_decode's
 * for the same q, tables and lengths (to rounding), per sequence:
 *     out[s, h] = softmax_t(scale * q[s, h] . K_s[t]) V_s[t] over its L_s tokens.
 *
 *   group_start    device int32 [num_groups + 1]: 0 = group_start[0] <= ... <=
 *                  group_start[num_groups] = num_seqs
 *   prefix_lens    device int32 [num_groups], 0 <= prefix_lens[j] <= every
 *                  member's length
 *   max_group_size host bound on every group's size
 *   other arguments as for pa_decode (block_size any positive value here)
 *   workspace      pa_decode_shared_prefix_workspace_size(...) bytes, 16-byte
 *                  aligned, no zero-fill needed (enough for either path below)
 *
 * A group is processed in blocks of 16 / (num_heads / num_kv_heads) members
 * (at most 16 query heads per KV head); each block reads the prefix once.
 * With block_size 8, 16 or 32, fewer than 2^22 blocks in the pool, at most
 * 2,048 such member blocks and laid-out tables of at most 256 MiB (bounded by
 * member blocks x (members per block + 1) x max_seq_len / block_size entries),
 * the call runs on pa_decode's kernels: a layout
 * kernel writes, for every member block, one table holding the prefix (rounded
 * down to whole 16-token units, or 32-token blocks) and then each member's own
 * tokens, each member's part starting on a whole unit; the decode kernel reads
 * those tables with the members as the rows of each (block, KV head) pair,
 * every row seeing the prefix and its own part only, the step split evenly
 * over the waves; the merge kernel folds pairs cut by a wave boundary.
 * Otherwise a multi-query kernel takes (group block, KV head, context
 * partition) items, longest group first, with a partition merge when there are
 * few items.  PA_SHARED_PREFIX_ROWS=0 selects the second path for every call.
 * float16 and bfloat16 only (PA_ERR_UNSUPPORTED for float32).  Index data that
 * breaks the contract is clamped so that no access leaves the arrays, with
 * unspecified results; PA_DEBUG_CHECK=1 rejects it, including tables that do
 * not share the stated prefix.  Results are deterministic.
 */
size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int num_groups, int num_heads,
                                              int num_kv_heads, int head_dim, int max_group_size,
                                              int max_seq_len);
pa_status pa_decode_shared_prefix(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens,
                                  int num_seqs, int num_groups, int num_heads, int num_kv_heads,
                                  int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_group_size, int max_seq_len, float scale, pa_dtype dtype,
                                  void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Swap blocks between two pools -- preemption ([PA-notes] §5 ③: when memory
 * runs short a request is suspended, its blocks freed or moved to CPU RAM, and
 * it is restored later through its block table).  For every (src, dst) row of
 * src_dst_pairs[num_pairs][2], block dst of the destination pool becomes a bit
 * copy of block src of the source pool, K and V, every slot and KV head.
 * Swap-out: source = the HBM pool, destination = a host pool; swap-in: the
 * reverse.  Both pools have the layout above with the same block_size,
 * num_kv_heads, head_dim and dtype, and src_num_blocks / dst_num_blocks blocks.
 *
 * Memory.  Unlike the other entry points, the pools and the pair array may be
 * device memory or pinned host memory allocated with hipHostMalloc (torch:
 * pin_memory=True); the kernel reads and writes host memory directly over the
 * host link, in one launch for all pairs.  Any other pointer (pageable host
 * memory) is refused with PA_ERR_INVALID before launching.  The two pools must
 * not overlap (identical base pointers are refused; use pa_copy_blocks within
 * one pool).  Repeated dst ids are invalid; pairs outside either pool are
 * skipped (PA_DEBUG_CHECK=1 rejects both).  The host must not touch a host
 * pool while a swap that uses it is in flight: synchronise the stream first.
 */
pa_status pa_swap_blocks(const void* src_k, const void* src_v, int src_num_blocks, void* dst_k,
                         void* dst_v, int dst_num_blocks, const int32_t* src_dst_pairs,
                         int num_pairs, int block_size, int num_kv_heads, int head_dim,
                         pa_dtype dtype, void* stream);

/*
 * Block manager -- host bookkeeping of the block pool ([PA-notes] §3 block
 * table; §5 ①② pool and on-demand allocation; §5 ③ swapping; §6.1, §6.2 and §12 题4 sharing,
 * reference counts and copy-on-write).
 *
 * It owns no device memory: it decides which physical block every token of
 * every sequence lives in and hands the kernels their index inputs -- block
 * tables and lengths (pa_bm_batch -> pa_decode), one slot per new token
 * (pa_bm_append_slot -> pa_write_kv) and copy-on-write pairs (-> pa_copy_blocks).
 * Every array here is HOST memory.  A manager is not thread-safe: use it from
 * one thread at a time.  On any non-PA_OK status the manager is unchanged.
 *
 * Rules: free blocks form a queue (taken from the front, released to the back;
 * the initial order is free_order, or 0..num_blocks-1).  A prompt of n tokens
 * takes ceil(n / block_size) blocks.  A new token goes to the next slot after
 * the filled ones of the sequence's last block, and a new block is taken only
 * when that block is full.  A fork shares every block of the parent (each
 * block's count goes up by one).  Writing into a block whose count is above one
 * first takes a fresh block, points only the writer's table at it, moves one
 * count from the old block to it and reports the (old, fresh) pair, whose
 * contents the caller copies with pa_copy_blocks before writing.  Freeing a
 * sequence decrements its blocks; a block whose count reaches zero returns to
 * the queue.  Sequences are named by any int64 id.
 */
typedef struct pa_block_manager pa_block_manager;

/* New manager of num_blocks GPU blocks of block_size tokens, plus a host pool
 * of num_cpu_blocks blocks for swapped-out sequences (0 = no swapping).
 * free_order: NULL or a host array holding a permutation of 0..num_blocks-1
 * (the host pool is handed out in id order). */
pa_status pa_bm_create(int num_blocks, int block_size, const int32_t* free_order,
                       int num_cpu_blocks, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* Prefill: give a new sequence ceil(num_tokens / block_size) blocks holding
 * num_tokens tokens.  PA_ERR_NO_BLOCKS if the pool is too small. */
pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq, int64_t num_tokens);

/* Reserve the slot of the sequence's next token: *slot = block * block_size +
 * offset.  If the write needs a private copy of a shared block, *cow_src and
 * *cow_dst name it (else both are -1). */
pa_status pa_bm_append_slot(pa_block_manager* bm, int64_t seq, int64_t* slot,
                            int32_t* cow_src, int32_t* cow_dst);

/* One decode step: reserve the next slot of each of the num_seqs distinct
 * sequences seqs[i], in that order, as pa_bm_append_slot does.  Writes
 * slot_mapping[i] (the pa_write_kv input) and the step's copy-on-write pairs to
 * pairs[2 * *num_pairs] as (src, dst) rows (the pa_copy_blocks input; at most
 * num_seqs rows, none of whose dst is a src).  Run pa_copy_blocks on the pairs
 * before pa_write_kv.  All or nothing: if the pool cannot supply every block
 * the step takes, returns PA_ERR_NO_BLOCKS and changes nothing.
 * PA_ERR_UNSUPPORTED if num_blocks * block_size does not fit int32 slots. */
pa_status pa_bm_append_step(pa_block_manager* bm, const int64_t* seqs, int num_seqs,
                            int32_t* slot_mapping, int32_t* pairs, int* num_pairs);

/* Parallel sampling / beam fork: `child` shares every block of `parent`. */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Drop a sequence (finished, or pruned from a beam). */
pa_status pa_bm_free(pa_block_manager* bm, int64_t seq);

/* Preemption ([PA-notes] §5 ③).  pa_bm_swap_out moves the listed sequences
 * (distinct, resident) to the host pool; pa_bm_swap_in brings the listed
 * (swapped-out) ones back into fresh GPU blocks.  The sequences of one call
 * move together: each distinct block they reference moves once, in order of
 * first reference, to the next free block of the target pool, and keeps its
 * count of listed sharers; a block also held by an unlisted sequence stays
 * where it is for that sequence.  The (src, dst) block pairs to copy with
 * pa_swap_blocks go to pairs[2 * *num_pairs] (pairs_cap rows available; the
 * sum of the listed tables' lengths always suffices).  Blocks released by the
 * move can be handed out again at once, so enqueue the copy before any later
 * write.  A swapped-out sequence can only be swapped in or freed.
 * PA_ERR_NO_BLOCKS if the target pool is short; nothing changes on error. */
pa_status pa_bm_swap_out(pa_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* pairs,
                         int pairs_cap, int* num_pairs);
pa_status pa_bm_swap_in(pa_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* pairs,
                        int pairs_cap, int* num_pairs);

int pa_bm_num_free(const pa_block_manager* bm);               /* -1 if bm is NULL */
int pa_bm_num_free_cpu(const pa_block_manager* bm);           /* host pool; -1 if bm is NULL */
int pa_bm_is_swapped(const pa_block_manager* bm, int64_t seq); /* 1, 0, or -1 if unknown */
int pa_bm_cpu_ref_count(const pa_block_manager* bm, int32_t block); /* -1 out of range */
int64_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq); /* -1 if unknown */
/* Copies up to cap entries of the sequence's table to out; returns its length
 * in blocks (-1 if unknown). */
int pa_bm_table(const pa_block_manager* bm, int64_t seq, int32_t* out, int cap);
int pa_bm_ref_count(const pa_block_manager* bm, int32_t block); /* -1 out of range */

/* Decode inputs for a batch: row i of block_tables[num_seqs][max_blocks_per_seq]
 * gets the table of seqs[i] padded with -1, seq_lens[i] its length.  Host
 * arrays; the caller copies them to the device. */
pa_status pa_bm_batch(const pa_block_manager* bm, const int64_t* seqs, int num_seqs,
                      int32_t* block_tables, int max_blocks_per_seq, int32_t* seq_lens);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
