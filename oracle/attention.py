"""Paged decode attention, plain float64 definition (oracle, test infrastructure).

What is computed
----------------
One decode step attends a single query per sequence to all of that sequence's
cached keys and values:  out = softmax(q·Kᵀ·scale)·V  ([vLLM-what]
"2）PagedAttention 算子", the dense formula with 1/√d; [PA-explainer]
"并行Attention计算" also divides by √d).  The paging changes only where K and V
sit: each sequence's tokens are cut into fixed-size logical blocks ([PA-notes]
§3, 16 tokens by default), every logical block lives in some physical block of
one shared pool, and a per-sequence block table gives logical -> physical
([PA-notes] §3; [vLLM-what] "2）PagedAttention 算子").  The softmax is
normalised over *all* tokens of the sequence, across blocks ([PA-notes] §4).

Readings where the pages are silent
--------------------------------------------------------------------
* Pool layout: ``cache[num_blocks, block_size, num_kv_heads, head_dim]``, the
  per-block ``[block_size, heads, head_dim]`` shape of [PA-explainer]
  "Block结构" with the KV heads of GQA ([vLLM-what] "1）KV cache 显存估算":
  Llama-3-8B keeps 8 KV heads, not 32).
* Token t (0-based) is in logical block t // B at offset t % B; the fill of the
  last block is implied by the sequence length.
* GQA: query head h reads KV head h // g with g = num_heads / num_kv_heads.
* ``scale`` is an explicit argument (1/√head_dim in every workload);
  [PA-notes] §4 writes the block scores without it.
* A sequence of length 0 attends to nothing and yields zeros.
* Table entries past ceil(L/B), and pool slots past a sequence's length, are
  never read.

``paged_multi_query`` extends the decode step to several query tokens per
sequence (chunked prefill, speculative verification): each query sees the
sequence's tokens up to and including its own position.

``attend`` is the two-pass stable softmax of the definition.  It deliberately is
*not* the blockwise online merge that the GPU uses, so the GPU's merge is
checked against a different algorithm.  ``paged_decode_blockwise`` is the
pages' own blockwise formulation ([PA-notes] §4): block scores S_ij, running
max / running sum merged block by block, O_i accumulated block by block.  It is
kept as a second oracle and pinned against the definition.

Pins (tests/test_oracle_attention.py): L = 1 returns v exactly; q = 0 returns
the mean of the valid V rows; a constructed one-hot attention returns the
selected row; a two-token case matches the logistic closed form; agreement
with torch's scaled_dot_product_attention in float64 on unpaged tensors (GQA by
repeating KV heads); bit-identical results under any relabelling of physical
block ids; blockwise == two-pass within 1e-12.  Multi-query
(tests/test_oracle_multi_query.py): one query per sequence equals the decode
oracle; agreement with torch's scaled_dot_product_attention in float64 under an
explicit causal mask offset by the cached prefix; the first query of a fresh
prompt returns V[0] exactly; changing K/V after a query's position leaves it
bit-identical while changing one at or before it does not.
"""

import numpy as np

from .dtypes import to_f64


def gather(cache, table_row, seq_len, block_size):
    """Contiguous ``[seq_len, num_kv_heads, head_dim]`` copy of one sequence.

    Token t is read from physical block ``table_row[t // block_size]`` at
    offset ``t % block_size`` ([PA-notes] §3 block table, §9.2 worked mapping).
    Only the first ceil(seq_len / block_size) table entries are used.
    """
    t = np.arange(seq_len)
    table_row = np.asarray(table_row)
    phys = table_row[t // block_size]
    return cache[phys, t % block_size]


def attend(q, K, V, scale):
    """Single-query attention for all query heads of one sequence, float64.

    q: [num_heads, head_dim]; K, V: [L, num_kv_heads, head_dim] (float64).
    Returns [num_heads, head_dim].  Query head h uses KV head h // g.
    """
    num_heads, head_dim = q.shape
    L, num_kv_heads, _ = K.shape
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    g = num_heads // num_kv_heads
    out = np.zeros((num_heads, head_dim), dtype=np.float64)
    if L == 0:
        return out
    for h in range(num_heads):
        kv = h // g
        s = scale * (K[:, kv, :] @ q[h])          # logits over all L tokens
        p = np.exp(s - s.max())                    # pass 1: max; pass 2: exp
        out[h] = (p @ V[:, kv, :]) / p.sum()
    return out


def paged_decode(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype, seqs=None):
    """Oracle for one paged decode step.

    q: [num_seqs, num_heads, head_dim]; k_cache, v_cache:
    [num_blocks, block_size, num_kv_heads, head_dim]; block_tables:
    [num_seqs, max_blocks_per_seq] int; seq_lens: [num_seqs] int.  Arrays are
    stored as ``dtype`` (bf16 as uint16 bits).  ``seqs`` optionally restricts the
    computation to some sequence indices (result rows in that order).
    Returns float64 [len(seqs), num_heads, head_dim].
    """
    block_size = k_cache.shape[1]
    seqs = range(q.shape[0]) if seqs is None else list(seqs)
    res = []
    for s in seqs:
        L = int(seq_lens[s])
        K = to_f64(gather(k_cache, block_tables[s], L, block_size), dtype)
        V = to_f64(gather(v_cache, block_tables[s], L, block_size), dtype)
        res.append(attend(to_f64(q[s], dtype), K, V, scale))
    return np.stack(res) if res else np.zeros((0,) + q.shape[1:])


def paged_multi_query(q, k_cache, v_cache, block_tables, seq_lens, q_start, scale, dtype):
    """Oracle for several query tokens per sequence over the paged cache, causal.

    The pages pair PagedAttention with chunked prefill (long prompts processed
    in pieces: [PA-explainer] "2026年最新进展"; the per-batch token cap for long
    prompts in [vLLM-what] "5）关键参数旋钮") and with speculative decoding
    ([PA-explainer] "2026年最新进展"), where a sequence brings several new
    tokens at once.  Sequence s owns the
    query rows ``q_start[s] .. q_start[s+1]-1``; they are its *last* n_s tokens
    (already written to the cache), so query i sits at position p = L_s - n_s + i
    and attends to the tokens 0..p of the sequence -- the dense causal definition,
    softmax(scale * q K[0..p]^T) V[0..p], with GQA as in ``attend``.

    q: [total_q, num_heads, head_dim]; seq_lens: [N] tokens in the cache
    including the queries' own; q_start: [N+1] non-decreasing offsets into q.
    Rows of q owned by no sequence stay zero.  Requires n_s <= L_s.
    Returns float64 [total_q, num_heads, head_dim].
    """
    block_size = k_cache.shape[1]
    q_start = [int(x) for x in q_start]
    total_q = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(len(seq_lens)):
        L = int(seq_lens[s])
        a, b = q_start[s], q_start[s + 1]
        n = b - a
        if n < 0 or b > total_q or a < 0:
            raise ValueError(f"sequence {s}: bad query range [{a}, {b})")
        if n > L:
            raise ValueError(f"sequence {s}: {n} queries but only {L} tokens")
        if n == 0:
            continue
        K = to_f64(gather(k_cache, block_tables[s], L, block_size), dtype)
        V = to_f64(gather(v_cache, block_tables[s], L, block_size), dtype)
        for i in range(n):
            pos = L - n + i
            out[a + i] = attend(to_f64(q[a + i], dtype), K[:pos + 1], V[:pos + 1], scale)
    return out


def paged_decode_blockwise(q, k_cache, v_cache, table_row, seq_len, scale, dtype):
    """The pages' blockwise formulation for one sequence ([PA-notes] §4).

    For each logical block j (tokens jB .. jB+B-1, clipped to the length) the
    block scores S_j = scale·q·K_jᵀ are merged into a running max m and a
    running sum ℓ, and the unnormalised output o is rescaled by exp(m_old -
    m_new) before adding exp(S_j - m_new)·V_j; the result is o / ℓ.  Physical
    blocks are fetched through ``table_row``.  float64 throughout.
    """
    block_size = k_cache.shape[1]
    qf = to_f64(q, dtype)
    num_heads, head_dim = qf.shape
    num_kv_heads = k_cache.shape[2]
    g = num_heads // num_kv_heads
    m = np.full(num_heads, -np.inf)
    l = np.zeros(num_heads)
    o = np.zeros((num_heads, head_dim))
    nblk = -(-seq_len // block_size)
    for j in range(nblk):
        n = min(block_size, seq_len - j * block_size)
        Kj = to_f64(k_cache[table_row[j], :n], dtype)
        Vj = to_f64(v_cache[table_row[j], :n], dtype)
        for h in range(num_heads):
            kv = h // g
            S = scale * (Kj[:, kv, :] @ qf[h])
            m_new = max(m[h], S.max())
            r = np.exp(m[h] - m_new)               # exp(-inf) = 0 on the first block
            P = np.exp(S - m_new)
            o[h] = o[h] * r + P @ Vj[:, kv, :]
            l[h] = l[h] * r + P.sum()
            m[h] = m_new
    out = np.zeros((num_heads, head_dim))
    if nblk:
        out = o / l[:, None]
    return out
