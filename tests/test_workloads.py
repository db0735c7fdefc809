"""The seeded workloads' host bookkeeping agrees with the reference block manager.

The workloads build block tables, write slots and copy-on-write pairs with their
own plain loops; replaying the same prompts, appends and forks through
``oracle.BlockManager`` with the same free-list order must give the same result.
Also checks the pool holds exactly the drawn rows at the table's slots and NaN
everywhere else.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import as_numpy


def replay_independent(b):
    bm = oracle.BlockManager(b.num_blocks, b.block_size, free_order=b.info["free_list"])
    N = b.num_seqs
    for s in range(N):
        bm.allocate(s, int(b.seq_lens_before[s]))
    slots = []
    for s in range(N):
        for _ in range(int(b.seq_lens[s]) - int(b.seq_lens_before[s])):
            slot, cow = bm.append_slot(s)
            assert cow is None
            slots.append(slot)
    return bm, slots


def check_tables(b, bm):
    for s in range(b.num_seqs):
        row = b.block_tables[s].tolist()
        n = len(bm.tables[s])
        assert row[:n] == bm.tables[s]
        assert all(x == -1 for x in row[n:])


@pytest.mark.parametrize("make", [
    lambda: workloads.tiny(),
    lambda: workloads.llama3_8b(num_seqs=12, num_blocks=3000),
    lambda: workloads.llama7b(num_seqs=6, max_len=300),
    lambda: workloads.llama2_70b(block_size=8, num_seqs=3, min_len=100, max_len=400),
    lambda: workloads.multi_query_small(),
    lambda: workloads.llama3_8b_spec(num_seqs=10, num_blocks=3000),
    lambda: workloads.llama3_8b_chunk(num_seqs=3, chunk=40, max_prior=100),
])
def test_independent_sequences_match_block_manager(make):
    b = make()
    bm, slots = replay_independent(b)
    check_tables(b, bm)
    if b.slot_mapping is not None:
        assert b.slot_mapping.tolist() == slots


def test_tiny_matches_the_stated_shape():
    b = workloads.tiny()
    assert b.seq_lens_before.tolist() == [1, 7, 16, 40]
    assert b.seq_lens.tolist() == [2, 8, 17, 41]
    assert b.num_blocks == 32 and b.block_size == 16 and b.head_dim == 64
    # the 16-token sequence needs a fresh block for its new token
    assert (b.block_tables[2] >= 0).sum() == 2


def test_shared_prefix_and_cow_match_block_manager():
    for cow in (False, True):
        if cow:
            b = workloads.opt13b_cow(num_prompts=3, samples=4, prompt_len=40)
        else:
            b = workloads.opt13b_shared(num_prompts=3, samples=4, prompt_len=32, tail_max=20)
        S = b.info["samples"]
        bm = oracle.BlockManager(b.num_blocks, b.block_size, free_order=b.info["free_list"])
        for p in range(b.num_seqs // S):
            bm.allocate(p * S, int(b.seq_lens_before[p * S]) - b.info["tails"][p * S])
        for p in range(b.num_seqs // S):
            for i in range(1, S):
                bm.fork(p * S, p * S + i)
        pairs, slots = [], []
        for s in range(b.num_seqs):
            extra = 1 if cow else b.info["tails"][s]
            for _ in range(extra):
                slot, c = bm.append_slot(s)
                slots.append(slot)
                if c is not None:
                    pairs.append(c)
        check_tables(b, bm)
        if cow:
            assert b.cow_pairs.tolist() == [list(p) for p in pairs]
            assert b.slot_mapping.tolist() == slots
            assert len(pairs) == 3 * (S - 1)


@pytest.mark.parametrize("make", [lambda: workloads.tiny(),
                                  lambda: workloads.opt13b_shared(num_prompts=2, samples=3,
                                                                  prompt_len=16, tail_max=9)])
def test_pool_holds_drawn_rows_and_nan_elsewhere(make):
    b = make()
    kc = as_numpy(b.k_cache).astype(np.float64)
    used = np.zeros(kc.shape[:2], bool)
    for s in range(b.num_seqs):
        L = int(b.seq_lens_before[s])
        for t in range(L):
            used[b.block_tables[s, t // b.block_size], t % b.block_size] = True
    assert np.isfinite(kc[used]).all()
    assert np.isnan(kc[~used]).all()


def test_draws_are_deterministic():
    a, b = workloads.tiny(seed=3), workloads.tiny(seed=3)
    assert torch.equal(a.q, b.q) and torch.equal(a.block_tables, b.block_tables)
    assert torch.equal(a.new_k, b.new_k)
    c = workloads.tiny(seed=4)
    assert not torch.equal(a.q, c.q)


def test_outliers_scale_key_rows_by_eight():
    b0 = workloads.llama2_70b(block_size=16, num_seqs=2, min_len=300, max_len=300,
                              outlier_frac=0.0)
    b1 = workloads.llama2_70b(block_size=16, num_seqs=2, min_len=300, max_len=300,
                              outlier_frac=0.01)
    # same draws up to the mask: each key row is either equal or exactly 8x
    k0 = oracle.to_f64(as_numpy(b0.k_cache), "bf16")
    k1 = oracle.to_f64(as_numpy(b1.k_cache), "bf16")
    fin = np.isfinite(k0[..., 0])
    rows0, rows1 = k0[fin], k1[fin]
    same = np.all(rows0 == rows1, axis=-1)
    eight = np.all(rows1 == 8 * rows0, axis=-1)
    assert np.all(same | eight) and 0 < (~same).sum() < 0.05 * same.size


def test_multi_query_batches_have_one_query_row_per_written_token():
    for b in (workloads.multi_query_small(), workloads.llama3_8b_chunk(num_seqs=3, chunk=40,
                                                                       max_prior=100)):
        n = (b.q_start[1:] - b.q_start[:-1]).tolist()
        assert b.q.shape[0] == sum(n) == len(b.slot_mapping)
        assert ((b.seq_lens - b.seq_lens_before).tolist()) == n
        assert all(k <= L for k, L in zip(n, b.seq_lens.tolist()))


@pytest.mark.parametrize("make", [lambda: workloads.opt13b_shared(num_prompts=3, samples=4, prompt_len=48,
                                                                  tail_max=30),
                                  lambda: workloads.opt13b_cow(num_prompts=3, samples=4, prompt_len=37)])
def test_shared_groups_really_share_their_prefix_blocks(make):
    b = make()
    B = b.block_size
    gs, P = b.group_start.tolist(), b.prefix_lens.tolist()
    assert gs[0] == 0 and gs[-1] == b.num_seqs and len(P) == len(gs) - 1
    tables, lens = b.block_tables.tolist(), b.seq_lens.tolist()
    for g in range(len(P)):
        nb = -(-P[g] // B)
        assert nb > 0
        for s in range(gs[g], gs[g + 1]):
            assert P[g] <= lens[s]
            assert tables[s][:nb] == tables[gs[g]][:nb]
