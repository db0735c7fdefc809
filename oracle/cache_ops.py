"""Cache writes and block copies, reference semantics (oracle, test infrastructure).

write_kv
    A newly generated token's K/V goes into the next free slot after the filled
    ones of its sequence's last block; a new physical block is taken only when
    that block is full ([PA-notes] §5 ②; [vLLM-what] "通俗解释": K/V of every
    generated token is written down for reuse).  The host hands the kernel the
    resulting slot per token: ``slot = physical_block * block_size + offset``,
    with a negative slot meaning "padding token, write nothing".  The slot
    encoding is not on the pages; it is the plainest flat index into the pool of
    [PA-notes] §3.  Two tokens naming the same slot in one call is invalid.

copy_blocks
    Copy-on-write: before a sequence writes into a physical block that other
    sequences still share, the block is duplicated and only the writer's table
    entry is repointed ([PA-notes] §6.1 and §12 题4).  The copy covers the whole
    block -- every slot, every KV head, K and V.  All pairs of one call are
    simultaneous (every read happens before any write); a pair with src == dst,
    a repeated dst, or a dst that is also some pair's src is invalid.

swap_blocks
    Preemption: when memory runs short a request is suspended, its blocks are
    released or moved to CPU RAM, and it is later restored through its block
    table ([PA-notes] §5 ③, likened there to OS paging).  The move is a block
    copy between two different pools (HBM and pinned host memory, either way):
    block ``dst`` of the destination pool := block ``src`` of the source pool,
    whole blocks, K and V.  A repeated dst is invalid; since the pools are
    distinct, a src may equal a dst id.

All three operations move bits and compute nothing, so the GPU must match them bit
for bit.  Pins (tests/test_oracle_cache_ops.py): the worked mapping of
[PA-notes] §9.2 (table [5, 2, 9]: token 40 goes to slot 152), targets equal
sources bit for bit, every other pool byte unchanged, invalid inputs rejected;
swap_blocks also through the block manager's swap traces
(tests/test_oracle_swap.py), where every sequence must read back its own tokens
after any mix of appends, forks, copies, swap-outs and swap-ins.
"""

import numpy as np


def _check_slots(slot_mapping, num_blocks, block_size):
    s = np.asarray(slot_mapping).astype(np.int64)
    live = s[s >= 0]
    if live.size and live.max() >= num_blocks * block_size:
        raise ValueError("slot beyond the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slot in one write")
    return s


def write_kv(k, v, slot_mapping, k_cache, v_cache):
    """Return copies of (k_cache, v_cache) with token i's rows stored at its slot.

    k, v: [num_tokens, num_kv_heads, head_dim]; caches:
    [num_blocks, block_size, num_kv_heads, head_dim], all the same storage type.
    """
    num_blocks, block_size = k_cache.shape[:2]
    slots = _check_slots(slot_mapping, num_blocks, block_size)
    kc = k_cache.copy()
    vc = v_cache.copy()
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        b, off = divmod(int(slot), block_size)
        kc[b, off] = k[i]
        vc[b, off] = v[i]
    return kc, vc


def check_pairs(pairs, num_blocks):
    """Validate copy-on-write (src, dst) pairs; returns them as an int64 [n, 2] array."""
    p = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if p.size == 0:
        return p
    if p.min() < 0 or p.max() >= num_blocks:
        raise ValueError("block id out of range")
    src, dst = p[:, 0], p[:, 1]
    if np.any(src == dst):
        raise ValueError("src == dst")
    if np.unique(dst).size != dst.size:
        raise ValueError("repeated dst")
    if np.intersect1d(src, dst).size:
        raise ValueError("a dst is also a src")
    return p


def copy_blocks(k_cache, v_cache, pairs):
    """Return copies of the caches with block dst := block src for every pair."""
    p = check_pairs(pairs, k_cache.shape[0])
    kc = k_cache.copy()
    vc = v_cache.copy()
    if p.size:
        ks = k_cache[p[:, 0]].copy()               # all reads first ...
        vs = v_cache[p[:, 0]].copy()
        kc[p[:, 1]] = ks                            # ... then all writes
        vc[p[:, 1]] = vs
    return kc, vc


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs):
    """Return copies of (dst_k, dst_v) with block dst := source block src for every
    (src, dst) pair; the source pools are not changed."""
    p = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("pools differ in block shape or storage type")
    kc = dst_k.copy()
    vc = dst_v.copy()
    if p.size == 0:
        return kc, vc
    if p[:, 0].min() < 0 or p[:, 0].max() >= src_k.shape[0]:
        raise ValueError("src block out of range")
    if p[:, 1].min() < 0 or p[:, 1].max() >= dst_k.shape[0]:
        raise ValueError("dst block out of range")
    if np.unique(p[:, 1]).size != len(p):
        raise ValueError("repeated dst")
    kc[p[:, 1]] = src_k[p[:, 0]]
    vc[p[:, 1]] = src_v[p[:, 0]]
    return kc, vc
