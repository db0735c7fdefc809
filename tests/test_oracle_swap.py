"""Pins for swapping blocks between the GPU pool and a host pool (preemption,
[PA-notes] §5 ③): ``oracle.swap_blocks`` and ``BlockManager.swap_out/swap_in``.

The trace test is the main pin.  It keeps, for every sequence, the plain list of
the tokens it has been given -- a model that knows nothing about blocks.  Both
pools are arrays of token tags.  Each step of a random trace (prefill, append,
fork, free, swap-out, swap-in, and refusals when a pool is short) is applied to
the manager, and the pairs it returns are applied to the pools with
``oracle.copy_blocks`` and ``oracle.swap_blocks``.  Afterwards every sequence
must read back exactly its own token list through its block table, from the
pool it lives in, and every reference count must equal the number of tables
holding the block.  A wrong pair, a missed copy, a count off by one or a block
freed too early puts a foreign tag into some sequence's read-back.
"""

import numpy as np
import pytest

import oracle
from oracle import BlockManager, OutOfBlocks


def test_swap_blocks_small_example():
    src_k = np.arange(2 * 2 * 1 * 2, dtype=np.float16).reshape(2, 2, 1, 2)
    src_v = -src_k
    dst_k = np.full((3, 2, 1, 2), 7, dtype=np.float16)
    dst_v = dst_k.copy()
    k, v = oracle.swap_blocks(src_k, src_v, dst_k, dst_v, [(1, 0), (0, 2)])
    assert k[0].tolist() == [[[4, 5]], [[6, 7]]] and k[2].tolist() == [[[0, 1]], [[2, 3]]]
    assert (k[1] == 7).all() and (v[0] == -src_k[1]).all() and (v[2] == -src_k[0]).all()
    assert (dst_k == 7).all()                      # inputs untouched
    # a src may carry the same id as a dst: the pools are distinct
    k, _ = oracle.swap_blocks(src_k, src_v, dst_k, dst_v, [(1, 1)])
    assert (k[1] == src_k[1]).all()


@pytest.mark.parametrize("pairs", [[(0, 0), (1, 0)], [(2, 0)], [(0, 3)], [(-1, 0)]])
def test_swap_blocks_rejects_invalid_pairs(pairs):
    a = np.zeros((2, 2, 1, 2), np.float16)
    b = np.zeros((3, 2, 1, 2), np.float16)
    with pytest.raises(ValueError):
        oracle.swap_blocks(a, a, b, b, pairs)


class Pools:
    """Token tags in a GPU pool and a host pool; -1 = never written."""

    def __init__(self, bm):
        B = bm.block_size
        self.B = B
        self.gpu = np.full((bm.num_blocks, B, 1, 1), -1, np.int64)
        self.cpu = np.full((max(bm.num_cpu_blocks, 1), B, 1, 1), -1, np.int64)

    def write(self, slot, tag):
        self.gpu[slot // self.B, slot % self.B] = tag

    def cow(self, pairs):
        self.gpu, _ = oracle.copy_blocks(self.gpu, self.gpu, pairs)

    def out(self, pairs):
        self.cpu, _ = oracle.swap_blocks(self.gpu, self.gpu, self.cpu, self.cpu, pairs)

    def back(self, pairs):
        self.gpu, _ = oracle.swap_blocks(self.cpu, self.cpu, self.gpu, self.gpu, pairs)


def check(bm, pools, hist):
    B = bm.block_size
    held = np.zeros(bm.num_blocks, int)
    held_cpu = np.zeros(max(bm.num_cpu_blocks, 1), int)
    for s, tokens in hist.items():
        pool = pools.cpu if s in bm.swapped else pools.gpu
        table = bm.tables[s]
        assert len(table) == -(-len(tokens) // B) and bm.lens[s] == len(tokens)
        got = [int(pool[table[t // B], t % B, 0, 0]) for t in range(len(tokens))]
        assert got == tokens, s
        for b in table:
            (held_cpu if s in bm.swapped else held)[b] += 1
    assert held.tolist() == bm.ref
    assert held_cpu[:bm.num_cpu_blocks].tolist() == bm.cpu_ref
    assert sorted(list(bm.free) + [b for b in range(bm.num_blocks) if bm.ref[b]]) == \
        list(range(bm.num_blocks))
    assert sorted(list(bm.cpu_free) + [b for b in range(bm.num_cpu_blocks) if bm.cpu_ref[b]]) == \
        list(range(bm.num_cpu_blocks))


@pytest.mark.parametrize("seed", range(6))
def test_swap_traces_read_back_every_sequence(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.choice([2, 4, 16]))
    NB, NC = int(rng.integers(12, 40)), int(rng.integers(4, 30))
    bm = BlockManager(NB, B, free_order=rng.permutation(NB), num_cpu_blocks=NC)
    pools = Pools(bm)
    hist, tag, ids = {}, [0], [0]
    counts = {"out": 0, "in": 0, "refused": 0, "cow": 0, "shared_out": 0}

    def new_tag():
        tag[0] += 1
        return tag[0]

    for step in range(400):
        live = [s for s in hist if s not in bm.swapped]
        away = [s for s in hist if s in bm.swapped]
        op = rng.integers(0, 7)
        try:
            if op == 0 or not hist:
                n = int(rng.integers(0, 3 * B + 1))
                table = bm.allocate(ids[0], n)
                toks = [new_tag() for _ in range(n)]
                for t, x in enumerate(toks):
                    pools.write(table[t // B] * B + t % B, x)
                hist[ids[0]] = toks
                ids[0] += 1
            elif op in (1, 2) and live:
                s = live[rng.integers(len(live))]
                slot, cow = bm.append_slot(s)
                if cow:
                    pools.cow([cow])
                    counts["cow"] += 1
                x = new_tag()
                pools.write(slot, x)
                hist[s] = hist[s] + [x]
            elif op == 3 and live:
                p = live[rng.integers(len(live))]
                bm.fork(p, ids[0])
                hist[ids[0]] = list(hist[p])
                ids[0] += 1
            elif op == 4 and hist:
                s = list(hist)[rng.integers(len(hist))]
                bm.free_seq(s)
                del hist[s]
            elif op == 5 and live:
                group = list(rng.choice(live, size=int(rng.integers(1, min(3, len(live)) + 1)),
                                        replace=False))
                group = [int(g) for g in group]
                shared = any(bm.ref[b] > 1 for g in group for b in bm.tables[g])
                pairs = bm.swap_out(group)
                pools.out(pairs)
                counts["out"] += 1
                counts["shared_out"] += shared
            elif op == 6 and away:
                group = [int(g) for g in rng.choice(away, size=int(rng.integers(1, len(away) + 1)),
                                                    replace=False)]
                pairs = bm.swap_in(group)
                pools.back(pairs)
                counts["in"] += 1
        except OutOfBlocks:
            counts["refused"] += 1
        check(bm, pools, hist)
    for s in list(hist):
        bm.free_seq(s)
    assert bm.num_free() == NB and len(bm.cpu_free) == NC
    assert counts["out"] and counts["in"] and counts["refused"] and counts["shared_out"]


def test_group_swap_moves_a_shared_block_once_and_keeps_outside_sharers():
    bm = BlockManager(8, 4, num_cpu_blocks=8)
    bm.allocate("p", 6)                            # blocks 0, 1 (1 half full)
    bm.fork("p", "a")
    bm.fork("p", "b")
    assert bm.ref[:2] == [3, 3]
    pairs = bm.swap_out(["a", "b"])                # both shared blocks, once each
    assert pairs == [(0, 0), (1, 1)] and bm.cpu_ref[:2] == [2, 2] and bm.ref[:2] == [1, 1]
    assert bm.tables["p"] == [0, 1] and bm.tables["a"] == bm.tables["b"] == [0, 1]
    with pytest.raises(ValueError):
        bm.append_slot("a")                        # swapped out
    with pytest.raises(ValueError):
        bm.swap_out(["a"])
    bm.free_seq("p")                               # GPU blocks 0, 1 return to the pool
    assert bm.num_free() == 8
    pairs = bm.swap_in(["b"])                      # b alone: fresh GPU copies, a keeps the host ones
    assert [src for src, _ in pairs] == [0, 1] and bm.cpu_ref[:2] == [1, 1]
    slot, cow = bm.append_slot("b")                # b's last block is private now
    assert cow is None


def test_swap_refusal_leaves_state_unchanged():
    bm = BlockManager(6, 4, num_cpu_blocks=2)
    bm.allocate("x", 12)                           # 3 blocks
    before = (list(bm.free), list(bm.ref), list(bm.cpu_free), list(bm.cpu_ref), dict(bm.tables))
    with pytest.raises(OutOfBlocks):
        bm.swap_out(["x"])
    assert (list(bm.free), list(bm.ref), list(bm.cpu_free), list(bm.cpu_ref), dict(bm.tables)) \
        == before and not bm.swapped
