"""Pins for the write and copy-on-write oracle (bit-exact data movement)."""

import json
import os

import numpy as np
import pytest

import oracle

with open(os.path.join(os.path.dirname(__file__), "golden", "block_examples.json")) as f:
    FORTY = json.load(f)["forty_tokens"]


def pool(rng, NB, B, H, D, dt=np.float16):
    return rng.standard_normal((NB, B, H, D)).astype(dt)


def test_worked_mapping_slots_and_next_write():
    # table [5, 2, 9]: token t lives at slot table[t // 16] * 16 + t % 16
    B = FORTY["page"]["block_size"]
    table = FORTY["page"]["physical"]
    for t, slot in FORTY["derived"]["token_slot"]:
        assert table[t // B] * B + t % B == slot
    # the written token 40 lands in block 9 at offset 8 and nowhere else
    rng = np.random.default_rng(0)
    kc, vc = pool(rng, 16, B, 2, 4), pool(rng, 16, B, 2, 4)
    k = rng.standard_normal((1, 2, 4)).astype(np.float16)
    v = rng.standard_normal((1, 2, 4)).astype(np.float16)
    slot = FORTY["derived"]["next_token_slot"]
    kc2, vc2 = oracle.write_kv(k, v, [slot], kc, vc)
    assert kc2[9, 8].tobytes() == k[0].tobytes() and vc2[9, 8].tobytes() == v[0].tobytes()
    other = np.ones(kc.shape[:2], bool)
    other[9, 8] = False
    assert kc2[other].tobytes() == kc[other].tobytes()
    assert vc2[other].tobytes() == vc[other].tobytes()
    # and the gathered 41-token sequence ends with it
    g = oracle.gather(kc2, table, 41, B)
    assert g[40].tobytes() == k[0].tobytes()


def test_write_is_a_bit_copy_and_skips_negative_slots():
    rng = np.random.default_rng(1)
    B, H, D = 8, 3, 5
    kc = rng.integers(0, 2**16, (6, B, H, D), dtype=np.uint16)      # bf16 bit patterns
    vc = rng.integers(0, 2**16, (6, B, H, D), dtype=np.uint16)
    k = rng.integers(0, 2**16, (4, H, D), dtype=np.uint16)
    v = rng.integers(0, 2**16, (4, H, D), dtype=np.uint16)
    slots = [13, -1, 47, 0]
    kc2, vc2 = oracle.write_kv(k, v, slots, kc, vc)
    touched = np.zeros((6, B), bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kc2[s // B, s % B], k[i])
        assert np.array_equal(vc2[s // B, s % B], v[i])
        touched[s // B, s % B] = True
    assert np.array_equal(kc2[~touched], kc[~touched])
    assert np.array_equal(vc2[~touched], vc[~touched])
    assert touched.sum() == 3


def test_write_rejects_duplicate_or_out_of_pool_slots():
    rng = np.random.default_rng(2)
    kc, vc = pool(rng, 2, 4, 1, 2), pool(rng, 2, 4, 1, 2)
    k = np.zeros((2, 1, 2), np.float16)
    with pytest.raises(ValueError):
        oracle.write_kv(k, k, [3, 3], kc, vc)
    with pytest.raises(ValueError):
        oracle.write_kv(k, k, [3, 8], kc, vc)


def test_copy_blocks_copies_whole_blocks_simultaneously():
    rng = np.random.default_rng(3)
    kc = rng.integers(0, 2**16, (10, 4, 2, 3), dtype=np.uint16)
    vc = rng.integers(0, 2**16, (10, 4, 2, 3), dtype=np.uint16)
    pairs = [(7, 1), (7, 4), (2, 9)]
    kc2, vc2 = oracle.copy_blocks(kc, vc, pairs)
    for s, d in pairs:
        assert np.array_equal(kc2[d], kc[s]) and np.array_equal(vc2[d], vc[s])
    rest = [b for b in range(10) if b not in (1, 4, 9)]
    assert np.array_equal(kc2[rest], kc[rest]) and np.array_equal(vc2[rest], vc[rest])
    # the inputs are not modified
    kc3, _ = oracle.copy_blocks(kc, vc, [])
    assert np.array_equal(kc3, kc)


@pytest.mark.parametrize("pairs", [[(3, 3)], [(1, 2), (3, 2)], [(1, 2), (2, 5)], [(0, 12)]])
def test_copy_blocks_rejects_invalid_pairs(pairs):
    kc = np.zeros((10, 2, 1, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, kc, pairs)
