"""Pins for the reference block manager (allocation, append, fork, copy-on-write, free)."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import BlockManager, OutOfBlocks

with open(os.path.join(os.path.dirname(__file__), "golden", "cow_trace.json")) as f:
    COW = json.load(f)["page"]
with open(os.path.join(os.path.dirname(__file__), "golden", "block_examples.json")) as f:
    BLOCKS = json.load(f)


def test_forty_token_request_on_blocks_5_2_9():
    page = BLOCKS["forty_tokens"]["page"]
    order = page["physical"] + [b for b in range(16) if b not in page["physical"]]
    bm = BlockManager(16, page["block_size"], free_order=order)
    assert bm.allocate("r", page["num_tokens"]) == page["physical"]
    assert bm.waste("r") == page["block_size"] - page["fills"][-1]
    # the next token still fits in block 9: no new block
    slot, cow = bm.append_slot("r")
    assert slot == BLOCKS["forty_tokens"]["derived"]["next_token_slot"] and cow is None
    assert bm.tables["r"] == page["physical"] and bm.num_free() == 13


def test_thousand_token_request():
    page = BLOCKS["thousand_tokens"]["page"]
    bm = BlockManager(100, page["block_size"])
    assert len(bm.allocate("r", page["num_tokens"])) == page["num_blocks"]
    assert bm.waste("r") == page["block_size"] - page["last_fill"]


def test_cow_trace_of_four_sharers():
    blk = COW["shared_block"]
    order = [blk] + [b for b in range(12) if b != blk]
    bm = BlockManager(12, 16, free_order=order)
    bm.allocate(1, 5)                              # one partly filled block: block 7
    for o in range(2, COW["sharers"] + 1):
        bm.fork(1, o)
    assert bm.ref[blk] == COW["ref_before"]
    slot, cow = bm.append_slot(COW["writer"])
    src, dst = cow
    assert src == blk and dst != blk
    assert bm.ref[blk] == COW["ref_shared_after"] and bm.ref[dst] == COW["ref_copy_after"]
    assert bm.tables[COW["writer"]] == [dst]
    for o in range(1, COW["sharers"] + 1):
        if o != COW["writer"]:
            assert bm.tables[o] == [blk]
    assert slot == dst * 16 + 5
    # outputs finish one by one; a block returns to the pool when its count reaches zero
    for o in (1, 2, 4):
        bm.free_seq(o)
    assert bm.ref[blk] == COW["freed_when_ref_reaches"] and blk in bm.free
    bm.free_seq(COW["writer"])
    assert bm.num_free() == 12


def test_last_sharer_writes_in_place():
    bm = BlockManager(20, 16)
    bm.allocate("p", 1000 % 16 + 16)               # two blocks, last half full
    for i in range(7):
        bm.fork("p", i)
    pairs = [bm.append_slot(i)[1] for i in range(7)]
    assert all(p is not None for p in pairs)
    assert bm.append_slot("p")[1] is None          # ref had dropped to 1


def test_full_shared_block_needs_no_copy():
    bm = BlockManager(10, 4)
    bm.allocate("a", 8)
    bm.fork("a", "b")
    slot, cow = bm.append_slot("b")
    assert cow is None and len(bm.tables["b"]) == 3 and bm.tables["b"][:2] == bm.tables["a"]


@pytest.mark.parametrize("seed", range(5))
def test_random_traffic_waste_below_one_block_and_no_leaks(seed):
    rng = np.random.default_rng(seed)
    B, NB = int(rng.choice([4, 8, 16])), 400
    bm = BlockManager(NB, B, free_order=rng.permutation(NB))
    live = []
    for step in range(300):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                name = f"s{step}"
                bm.allocate(name, int(rng.integers(0, 40)))
                live.append(name)
            elif op == 1:
                bm.append_slot(live[rng.integers(len(live))])
            elif op == 2:
                child = f"f{step}"
                bm.fork(live[rng.integers(len(live))], child)
                live.append(child)
            else:
                bm.free_seq(live.pop(rng.integers(len(live))))
        except OutOfBlocks:
            pass
        for s in live:
            assert 0 <= bm.waste(s) < B or bm.lens[s] == 0
        # every reference is accounted for
        held = np.zeros(NB, int)
        for s in live:
            for b in bm.tables[s]:
                held[b] += 1
        assert held.tolist() == bm.ref
        assert sorted(list(bm.free) + [b for b in range(NB) if bm.ref[b]]) == list(range(NB))
    for s in list(live):
        bm.free_seq(s)
    assert bm.num_free() == NB and sum(bm.ref) == 0


def test_exhaustion_leaves_state_unchanged():
    bm = BlockManager(3, 4)
    bm.allocate("a", 8)
    before = (list(bm.free), list(bm.ref), {k: list(v) for k, v in bm.tables.items()})
    with pytest.raises(OutOfBlocks):
        bm.allocate("b", 9)
    assert (list(bm.free), list(bm.ref), {k: list(v) for k, v in bm.tables.items()}) == before
    bm.allocate("c", 4)
    bm.fork("c", "d")
    with pytest.raises(OutOfBlocks):
        bm.append_slot("d")        # needs a new block, none left
    assert bm.lens["d"] == 4 and bm.tables["d"] == bm.tables["c"]
