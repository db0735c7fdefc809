"""Seeded synthetic inputs for paged decode attention.

This module is the only code that both the HIP path's callers and the oracle's
callers use.  It draws random numbers and lays them out; it computes no
attention, softmax or copy arithmetic.  Everything is drawn on the CPU with a
``torch.Generator`` seeded per workload, in float32 from N(0, 1), then rounded
to the storage type (round-to-nearest-even, torch's conversion).

Host bookkeeping done here, in the order the pages give it ([PA-notes]
"LLM 注意力与计算内核精读笔记 · 05 PagedAttention 与 KV 显存管理" §3, §5, §6):
the free list is a seeded permutation of all physical ids; every sequence's
prompt takes ceil(n / B) blocks from the head of the list, sequences in order;
tokens appended afterwards go to the next slot of their last block, a new block
being taken only when it is full; parallel samples share their prompt's blocks;
a write into a shared, partly filled block first copies it (copy-on-write).
The slot of token t is ``table[t // B] * B + t % B``.

Draw order (fixed): lengths -> free-list permutation -> q -> K rows (all
sequences, sequence-major, as one [sum L, Hkv, D] draw) -> key outlier mask ->
V rows.  The last token of a sequence that arrives by a write step is a row of
that same draw; it is kept out of the pool and handed to the write instead.
Pool slots that hold no token are filled with NaN by default, so any read of
them poisons the result.

Workloads (shapes of the pages' examples):
  tiny            fp32, 4 seqs {1,7,16,40} + 1 written token each, B=16, 32 blocks
  worked_5_2_9    the 40-token request on physical blocks 5, 2, 9
  llama7b         MHA 32 heads, D=128, fp16, 64 seqs, L ~ U{1..2048}
  llama3_8b       GQA 32/8, D=128, bf16, 256 seqs, L ~ U{512..4096}, 70,000 blocks,
                  last token of each sequence written by the write step
  opt13b_shared   MHA 40 heads, fp16, 32 prompts x 8 samples sharing 64 blocks,
                  private tails U{0..256}
  opt13b_cow      same shape, 1000-token prompts (last block half full): the next
                  token of 7 of the 8 samples forces a block copy
  llama2_70b      GQA 64/8, D=128, bf16, 32 seqs, L ~ U{8192..32768},
                  B in {8,16,32}, 1% of key rows x8
  llama3_8b_spec  multi-query: the llama3_8b shape with 4 new tokens per sequence
  llama3_8b_chunk multi-query: 16 sequences x 512-token prompt chunks after cached
                  prefixes of U{0..3584} tokens
Every size parameter can be shrunk for oracle-sized parity cases.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class PagedBatch:
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    q: torch.Tensor                      # [N, Hq, D]
    k_cache: torch.Tensor                # [NB, B, Hkv, D]
    v_cache: torch.Tensor
    block_tables: torch.Tensor           # int32 [N, MB], -1 past each sequence's blocks
    seq_lens: torch.Tensor               # int32 [N]: tokens attention runs over
    seq_lens_before: torch.Tensor        # int32 [N]: tokens in the pool before the write step
    new_k: Optional[torch.Tensor] = None  # [T, Hkv, D] tokens of the write step
    new_v: Optional[torch.Tensor] = None
    slot_mapping: Optional[torch.Tensor] = None   # int32 [T]
    cow_pairs: Optional[torch.Tensor] = None      # int32 [P, 2] (src, dst) before the write
    q_start: Optional[torch.Tensor] = None        # int32 [N+1]: multi-query batches only
    group_start: Optional[torch.Tensor] = None    # int32 [G+1]: sequences sharing a prefix
    prefix_lens: Optional[torch.Tensor] = None    # int32 [G]: tokens in shared blocks
    info: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return int(self.seq_lens.shape[0])

    @property
    def max_q_len(self):
        if self.q_start is None:
            return 1
        d = self.q_start[1:] - self.q_start[:-1]
        return int(d.max()) if d.numel() else 0

    def causal_pairs(self):
        """Multi-query batches: sum over query rows of the tokens each attends to."""
        qs, lens = self.q_start.tolist(), self.seq_lens.tolist()
        tot = 0
        for s, L in enumerate(lens):
            n = qs[s + 1] - qs[s]
            tot += n * (L - n) + n * (n + 1) // 2
        return tot

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.num_seqs else 0

    def kv_bytes(self):
        """K and V bytes attention reads: each (token, KV head) row of K and V once."""
        esize = torch.empty((), dtype=TORCH_DTYPE[self.dtype]).element_size()
        return int(self.seq_lens.sum()) * self.num_kv_heads * self.head_dim * 2 * esize


def as_numpy(t):
    """numpy view of a CPU tensor in the oracle's storage convention (bf16 -> uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _round(x, dtype):
    return x.to(TORCH_DTYPE[dtype])


def _tables(prompt_lens, appended, block_size, free_list):
    """Block tables for sequences that first take ceil(prompt/B) blocks, all sequences in
    order, then append ``appended[s]`` tokens each (sequences in order).  Returns the
    tables (lists) and the index of the next unused free-list entry."""
    B = block_size
    nxt = 0
    tables = []
    for n in prompt_lens:
        k = -(-int(n) // B)
        tables.append([int(b) for b in free_list[nxt:nxt + k]])
        nxt += k
    for s, extra in enumerate(appended):
        pos = int(prompt_lens[s])
        for _ in range(int(extra)):
            if pos // B == len(tables[s]):
                tables[s].append(int(free_list[nxt]))
                nxt += 1
            pos += 1
    return tables, nxt


def _table_tensor(tables):
    mb = max(1, max((len(t) for t in tables), default=1))
    bt = torch.full((len(tables), mb), -1, dtype=torch.int32)
    for s, t in enumerate(tables):
        if t:
            bt[s, :len(t)] = torch.tensor(t, dtype=torch.int32)
    return bt


def _slots(table, start, stop, B):
    t = torch.arange(start, stop, dtype=torch.int64)
    tab = torch.tensor(table, dtype=torch.int64) if table else torch.zeros(1, dtype=torch.int64)
    return tab[t // B] * B + t % B


def _pool(num_blocks, B, Hkv, D, dtype, fill):
    val = float("nan") if fill == "nan" else 0.0
    return torch.full((num_blocks, B, Hkv, D), val, dtype=TORCH_DTYPE[dtype])


def _paged(*, name, dtype, lens, Hq, Hkv, D, B, num_blocks=None, slack=0.10, gen,
           write_last=False, outlier_frac=0.0, fill="nan", queries=None):
    """Independent sequences: prompts of L-1 (write_last) or L tokens, random placement.

    With ``queries`` (tokens per sequence), the last queries[s] tokens of every
    sequence arrive through the write step and each of them has a query row
    (several queries per sequence, causal); q is then [sum(queries), Hq, D]."""
    lens = [int(x) for x in lens]
    N = len(lens)
    if queries is not None:
        queries = [int(x) for x in queries]
        if any(n > L for n, L in zip(queries, lens)):
            raise ValueError(f"{name}: more queries than tokens")
        appended = queries
    else:
        appended = [1 if write_last else 0 for _ in lens]
    prompt = [L - a for L, a in zip(lens, appended)]
    need = sum(-(-L // B) for L in lens)
    if num_blocks is None:
        num_blocks = max(1, int(np.ceil(need * (1.0 + slack))))
    if need > num_blocks:
        raise ValueError(f"{name}: pool of {num_blocks} blocks cannot hold {need}")
    perm = torch.randperm(num_blocks, generator=gen).tolist()
    tables, _ = _tables(prompt, appended, B, perm)
    q = torch.randn(N if queries is None else sum(queries), Hq, D, generator=gen)
    total = sum(lens)
    K = torch.randn(total, Hkv, D, generator=gen)
    if outlier_frac > 0:
        mask = torch.rand(total, Hkv, generator=gen) < outlier_frac
        K[mask] *= 8.0                      # exact in every storage type
    V = torch.randn(total, Hkv, D, generator=gen)
    K, V, q = _round(K, dtype), _round(V, dtype), _round(q, dtype)
    kc = _pool(num_blocks, B, Hkv, D, dtype, fill)
    vc = _pool(num_blocks, B, Hkv, D, dtype, fill)
    kflat, vflat = kc.view(-1, Hkv, D), vc.view(-1, Hkv, D)
    new_rows, new_slots = [], []
    off = 0
    for s, L in enumerate(lens):
        stored = prompt[s]
        sl = _slots(tables[s], 0, stored, B)
        kflat[sl] = K[off:off + stored]
        vflat[sl] = V[off:off + stored]
        if appended[s]:
            new_rows.extend(range(off + stored, off + L))
            new_slots.extend(int(x) for x in _slots(tables[s], stored, L, B))
        off += L
    b = PagedBatch(
        name=name, dtype=dtype, num_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
        num_blocks=num_blocks, scale=1.0 / float(np.sqrt(D)), q=q, k_cache=kc, v_cache=vc,
        block_tables=_table_tensor(tables), seq_lens=torch.tensor(lens, dtype=torch.int32),
        seq_lens_before=torch.tensor(prompt, dtype=torch.int32),
        info={"blocks_needed": need, "free_list": perm})
    if new_rows:
        idx = torch.tensor(new_rows, dtype=torch.int64)
        b.new_k, b.new_v = K[idx].clone(), V[idx].clone()
        b.slot_mapping = torch.tensor(new_slots, dtype=torch.int32)
    if queries is not None:
        b.q_start = torch.tensor(np.concatenate([[0], np.cumsum(queries)]), dtype=torch.int32)
    return b


# --------------------------------------------------------------------------------------
# The workloads


def tiny(seed=0, fill="nan"):
    """fp32, 4 sequences of {1,7,16,40} tokens, one new token each via the write step."""
    g = torch.Generator().manual_seed(seed)
    return _paged(name="tiny", dtype="f32", lens=[2, 8, 17, 41], Hq=4, Hkv=4, D=64, B=16,
                  num_blocks=32, gen=g, write_last=True, fill=fill)


def worked_5_2_9(seed=0, dtype="f32", num_heads=4, num_kv_heads=4, head_dim=64, fill="nan"):
    """The 40-token request of the worked example on physical blocks 5, 2, 9, pool of 16
    blocks, plus one written token (position 40, which still fits in block 9)."""
    g = torch.Generator().manual_seed(seed)
    B, L = 16, 41
    table = [5, 2, 9]
    q = _round(torch.randn(1, num_heads, head_dim, generator=g), dtype)
    K = _round(torch.randn(L, num_kv_heads, head_dim, generator=g), dtype)
    V = _round(torch.randn(L, num_kv_heads, head_dim, generator=g), dtype)
    kc = _pool(16, B, num_kv_heads, head_dim, dtype, fill)
    vc = _pool(16, B, num_kv_heads, head_dim, dtype, fill)
    sl = _slots(table, 0, L - 1, B)
    kc.view(-1, num_kv_heads, head_dim)[sl] = K[:L - 1]
    vc.view(-1, num_kv_heads, head_dim)[sl] = V[:L - 1]
    return PagedBatch(
        name="worked_5_2_9", dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=B, num_blocks=16, scale=1.0 / float(np.sqrt(head_dim)),
        q=q, k_cache=kc, v_cache=vc, block_tables=torch.tensor([table], dtype=torch.int32),
        seq_lens=torch.tensor([L], dtype=torch.int32),
        seq_lens_before=torch.tensor([L - 1], dtype=torch.int32),
        new_k=K[L - 1:].clone(), new_v=V[L - 1:].clone(),
        slot_mapping=_slots(table, L - 1, L, B).to(torch.int32))


def llama7b(seed=0, num_seqs=64, min_len=1, max_len=2048, fill="nan"):
    """LLaMA-7B-shaped layer: 32 heads = 32 KV heads, D=128, fp16, B=16, pool = need + 10%."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(min_len, max_len + 1, (num_seqs,), generator=g).tolist()
    return _paged(name="llama7b", dtype="f16", lens=lens, Hq=32, Hkv=32, D=128, B=16,
                  gen=g, fill=fill)


def llama3_8b(seed=0, num_seqs=256, min_len=512, max_len=4096, num_blocks=70_000, fill="nan"):
    """Llama-3-8B-shaped GQA layer: 32 query / 8 KV heads, D=128, bf16, B=16, 70,000-block
    pool; each sequence's last token arrives through the write step (num_seqs tokens)."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(min_len, max_len + 1, (num_seqs,), generator=g).tolist()
    return _paged(name="llama3_8b", dtype="bf16", lens=lens, Hq=32, Hkv=8, D=128, B=16,
                  num_blocks=num_blocks, gen=g, write_last=True, fill=fill)


def llama2_70b(seed=0, block_size=16, num_seqs=32, min_len=8192, max_len=32768,
               outlier_frac=0.01, fill="nan"):
    """Llama-2-70B per-layer shape: 64 query / 8 KV heads, D=128, bf16, long contexts,
    1% of key rows scaled by 8, pool = need + 10%."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(min_len, max_len + 1, (num_seqs,), generator=g).tolist()
    return _paged(name=f"llama2_70b_b{block_size}", dtype="bf16", lens=lens, Hq=64, Hkv=8,
                  D=128, B=block_size, gen=g, outlier_frac=outlier_frac, fill=fill)


def llama3_8b_spec(seed=0, num_seqs=256, queries=4, min_len=512, max_len=4096,
                   num_blocks=70_000, fill="nan"):
    """Speculative verification on the Llama-3-8B shape: every sequence brings ``queries``
    new tokens (written by the write step), each scored against the whole cached context
    causally; lengths, including the new tokens, uniform in [min_len, max_len]."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(min_len, max_len + 1, (num_seqs,), generator=g).tolist()
    return _paged(name="llama3_8b_spec", dtype="bf16", lens=lens, Hq=32, Hkv=8, D=128, B=16,
                  num_blocks=num_blocks, gen=g, queries=[queries] * num_seqs, fill=fill)


def llama3_8b_chunk(seed=0, num_seqs=16, chunk=512, max_prior=3584, fill="nan"):
    """Chunked prefill on the Llama-3-8B shape: every sequence brings a ``chunk``-token
    piece of its prompt after a cached prefix of U{0..max_prior} tokens."""
    g = torch.Generator().manual_seed(seed)
    prior = torch.randint(0, max_prior + 1, (num_seqs,), generator=g).tolist()
    lens = [p + chunk for p in prior]
    return _paged(name="llama3_8b_chunk", dtype="bf16", lens=lens, Hq=32, Hkv=8, D=128, B=16,
                  gen=g, queries=[chunk] * num_seqs, fill=fill)


def multi_query_small(seed=0, dtype="f32", lens=(1, 7, 16, 40, 64, 33), queries=(1, 3, 16, 5, 64, 33),
                      Hq=8, Hkv=2, D=64, B=16, fill="nan"):
    """Oracle-sized multi-query batch: single queries, short and whole-prompt chunks."""
    g = torch.Generator().manual_seed(seed)
    return _paged(name=f"multi_query_small_{dtype}", dtype=dtype, lens=list(lens), Hq=Hq,
                  Hkv=Hkv, D=D, B=B, gen=g, queries=list(queries), fill=fill)


def _shared(*, name, seed, num_prompts, samples, prompt_len, tail_max, cow, Hq, D, B, fill):
    """Parallel sampling: every prompt's blocks are shared by ``samples`` sequences.

    Without ``cow`` each sample then appends a private tail of U{0..tail_max} tokens.
    With ``cow`` there are no tails; instead every sample's next token is written by the
    write step, and a write into the still-shared, partly filled last prompt block makes
    the writer copy it first (all but the last writer of each prompt)."""
    g = torch.Generator().manual_seed(seed)
    Hkv = Hq
    N = num_prompts * samples
    if cow:
        tails = [0] * N
    else:
        tails = torch.randint(0, tail_max + 1, (N,), generator=g).tolist()
    pblk = -(-prompt_len // B)
    partial = prompt_len % B != 0
    # private blocks: tail blocks, or copy-on-write targets
    if cow:
        priv = [(1 if (partial and (s % samples) != samples - 1) else 0)
                + (1 if not partial else 0) for s in range(N)]
    else:
        priv = [-(-max(0, t - (pblk * B - prompt_len)) // B) for t in tails]
    need = num_prompts * pblk + sum(priv)
    num_blocks = int(np.ceil(need * 1.10))
    perm = torch.randperm(num_blocks, generator=g).tolist()
    nxt = 0
    prompt_tables = []
    for _ in range(num_prompts):
        prompt_tables.append(perm[nxt:nxt + pblk])
        nxt += pblk
    tables = [list(prompt_tables[s // samples]) for s in range(N)]
    cow_pairs = []
    new_slots = []
    seq_lens_before = [prompt_len + t for t in tails]
    for s in range(N):
        pos = prompt_len
        extra = 1 if cow else tails[s]
        for i in range(extra):
            last_is_shared_partial = (pos // B < len(tables[s])) and pos // B == pblk - 1
            if pos // B == len(tables[s]):
                tables[s].append(perm[nxt]); nxt += 1
            elif last_is_shared_partial and cow and (s % samples) != samples - 1:
                src = tables[s][pos // B]
                tables[s][pos // B] = perm[nxt]; nxt += 1
                cow_pairs.append((src, tables[s][pos // B]))
            elif last_is_shared_partial and not cow:
                raise AssertionError("tails only start on a full prompt")
            if cow:
                new_slots.append(tables[s][pos // B] * B + pos % B)
            pos += 1
    assert nxt <= num_blocks
    q = _round(torch.randn(N, Hq, D, generator=g), "f16")
    Kp = _round(torch.randn(num_prompts * prompt_len, Hkv, D, generator=g), "f16")
    Vp = _round(torch.randn(num_prompts * prompt_len, Hkv, D, generator=g), "f16")
    ntail = sum(tails) + (N if cow else 0)
    Kt = _round(torch.randn(ntail, Hkv, D, generator=g), "f16")
    Vt = _round(torch.randn(ntail, Hkv, D, generator=g), "f16")
    kc = _pool(num_blocks, B, Hkv, D, "f16", fill)
    vc = _pool(num_blocks, B, Hkv, D, "f16", fill)
    kflat, vflat = kc.view(-1, Hkv, D), vc.view(-1, Hkv, D)
    for p in range(num_prompts):
        sl = _slots(prompt_tables[p], 0, prompt_len, B)
        kflat[sl] = Kp[p * prompt_len:(p + 1) * prompt_len]
        vflat[sl] = Vp[p * prompt_len:(p + 1) * prompt_len]
    off = 0
    if not cow:
        for s in range(N):
            sl = _slots(tables[s], prompt_len, prompt_len + tails[s], B)
            kflat[sl] = Kt[off:off + tails[s]]
            vflat[sl] = Vt[off:off + tails[s]]
            off += tails[s]
    lens = [prompt_len + t + (1 if cow else 0) for t in tails]
    b = PagedBatch(
        name=name, dtype="f16", num_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
        num_blocks=num_blocks, scale=1.0 / float(np.sqrt(D)), q=q, k_cache=kc, v_cache=vc,
        block_tables=_table_tensor(tables), seq_lens=torch.tensor(lens, dtype=torch.int32),
        seq_lens_before=torch.tensor(seq_lens_before, dtype=torch.int32),
        info={"blocks_needed": need, "free_list": perm, "samples": samples,
              "prompt_tables": prompt_tables, "tails": tails})
    if cow:
        b.new_k, b.new_v = Kt, Vt
        b.slot_mapping = torch.tensor(new_slots, dtype=torch.int32)
        b.cow_pairs = torch.tensor(cow_pairs, dtype=torch.int32).reshape(-1, 2)
    # the samples of a prompt are contiguous and share the prompt's blocks: all of
    # them, or (after copy-on-write of a partly filled last block) its full blocks
    shared = prompt_len if not (cow and partial) else (prompt_len // B) * B
    b.group_start = torch.arange(0, N + 1, samples, dtype=torch.int32)
    b.prefix_lens = torch.full((num_prompts,), shared, dtype=torch.int32)
    return b


def opt13b_shared(seed=0, num_prompts=32, samples=8, prompt_len=1024, tail_max=256, fill="nan"):
    """OPT-13B shape (40 heads = 40 KV heads, D=128, fp16, B=16): 32 prompts of 1024
    tokens, each sampled 8 ways sharing the prompt's 64 blocks, private tails U{0..256}."""
    return _shared(name="opt13b_shared", seed=seed, num_prompts=num_prompts, samples=samples,
                   prompt_len=prompt_len, tail_max=tail_max, cow=False, Hq=40, D=128, B=16,
                   fill=fill)


def opt13b_cow(seed=0, num_prompts=32, samples=8, prompt_len=1000, fill="nan"):
    """Copy-on-write variant: 1000-token prompts (63 blocks, last one 8/16 full) shared by
    8 samples; each sample's next token is written, so 7 of 8 samples copy the shared
    last block first.  Attention then runs over 1001 tokens."""
    return _shared(name="opt13b_cow", seed=seed, num_prompts=num_prompts, samples=samples,
                   prompt_len=prompt_len, tail_max=0, cow=True, Hq=40, D=128, B=16, fill=fill)


WORKLOADS = {
    "tiny": tiny,
    "llama7b": llama7b,
    "llama3_8b": llama3_8b,
    "opt13b_shared": opt13b_shared,
    "opt13b_cow": opt13b_cow,
    "llama2_70b": llama2_70b,
    "llama3_8b_spec": llama3_8b_spec,
    "llama3_8b_chunk": llama3_8b_chunk,
}
