"""GPU parity: the HIP path through the C-ABI against the float64 oracle.

Attention outputs must agree within max-abs 1e-5 (fp32), 4e-3 (fp16), 8e-3 (bf16);
writes and block copies must agree bit for bit over the whole pool.  Pools are
NaN-filled wherever no token lives, so a read past a sequence end, through a
padding table entry or from an unused block poisons the output.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import as_numpy, PagedBatch, TORCH_DTYPE
from _gpu import (TOL, assert_close, bits, gpu_decode, log, oracle_decode, pk, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk()


def random_batch(seed, dtype, lens, Hq, Hkv, D, B, extra=5):
    """Small paged batch in the workloads' recipe (random placement, NaN-filled pool)."""
    g = torch.Generator().manual_seed(seed)
    return workloads._paged(name=f"rand{seed}", dtype=dtype, lens=lens, Hq=Hq, Hkv=Hkv, D=D, B=B,
                            num_blocks=sum(-(-L // B) for L in lens) + extra, gen=g)


# ---------------------------------------------------------------------------- tiny


def test_tiny_config_write_and_decode():
    b = workloads.tiny()
    d = to_dev(b)
    m = pk()
    log("tiny: decode before write")
    got = gpu_decode(b, d, lens=d.lens_before)
    ref = oracle_decode(b, lens=b.seq_lens_before)
    assert_close(got, ref, "f32", "tiny before write")
    log("tiny: pa_write_kv of 4 tokens")
    m.pa_write_kv(d.new_k, d.new_v, d.slots, d.kc, d.vc)
    torch.cuda.synchronize()
    kc2, vc2 = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(b.slot_mapping),
                               as_numpy(b.k_cache), as_numpy(b.v_cache))
    assert torch.equal(bits(d.kc.cpu()), bits(torch.from_numpy(kc2)))
    assert torch.equal(bits(d.vc.cpu()), bits(torch.from_numpy(vc2)))
    log("tiny: decode after write")
    got = gpu_decode(b, d)
    ref = oracle.paged_decode(as_numpy(b.q), kc2, vc2, as_numpy(b.block_tables),
                              as_numpy(b.seq_lens), b.scale, "f32")
    assert_close(got, ref, "f32", "tiny after write")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_worked_example_5_2_9(dtype):
    b = workloads.worked_5_2_9(dtype=dtype, num_heads=8, num_kv_heads=2, head_dim=128)
    d = to_dev(b)
    log(f"worked_5_2_9 {dtype}")
    pk().pa_write_kv(d.new_k, d.new_v, d.slots, d.kc, d.vc)
    torch.cuda.synchronize()
    assert b.slot_mapping.tolist() == [152]
    kc2, vc2 = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), [152],
                               as_numpy(b.k_cache), as_numpy(b.v_cache))
    assert torch.equal(bits(d.kc.cpu()), bits(torch.from_numpy(kc2)))
    got = gpu_decode(b, d)
    ref = oracle.paged_decode(as_numpy(b.q), kc2, vc2, [[5, 2, 9]], [41], b.scale, dtype)
    assert_close(got, ref, dtype, "worked example")


# ---------------------------------------------------------------------------- special cases


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (16, 2), (12, 4)])
def test_single_token_returns_v_exactly(dtype, Hq, Hkv):
    b = random_batch(11, dtype, [1, 1, 17, 1], Hq, Hkv, 128, 16)
    d = to_dev(b)
    log(f"single token {dtype} {Hq}/{Hkv}")
    got = gpu_decode(b, d)
    g = Hq // Hkv
    for s in (0, 1, 3):
        slot = int(b.block_tables[s, 0]) * b.block_size
        v = b.v_cache.view(-1, Hkv, 128)[slot].double().numpy()
        for h in range(Hq):
            assert np.array_equal(got[s, h], v[h // g])


def test_empty_sequences_give_zeros():
    b = random_batch(12, "bf16", [0, 5, 0, 600], 8, 2, 128, 16)
    d = to_dev(b)
    log("empty sequences")
    got = gpu_decode(b, d)
    assert np.array_equal(got[0], np.zeros_like(got[0])) and np.array_equal(got[2], got[0] * 0)
    assert_close(got, oracle_decode(b), "bf16", "empty")


def test_all_sequences_empty():
    b = random_batch(13, "f16", [0, 0], 4, 4, 64, 8)
    d = to_dev(b)
    log("all empty")
    got = gpu_decode(b, d, max_seq_len=0)
    assert np.array_equal(got, np.zeros_like(got))


# ---------------------------------------------------------------------------- shape sweep

SWEEP = [(dt, D, B, Hq, Hkv)
         for dt in ("f32", "f16", "bf16")
         for D in (64, 128)
         for B in (8, 16, 32)
         for (Hq, Hkv) in ((4, 4), (6, 2), (8, 2), (16, 2), (16, 1))]


@pytest.mark.parametrize("dt,D,B,Hq,Hkv", SWEEP)
def test_shape_sweep(dt, D, B, Hq, Hkv):
    # lengths: one token, partial tiles, exact tile and block multiples, longer ones
    # with a ragged tail; the batch is small, so its pairs are split over many waves
    lens = [1, 3, 15, 16, 17, B, B + 1, 33, 511, 512, 513, 1031]
    b = random_batch(100 + SWEEP.index((dt, D, B, Hq, Hkv)), dt, lens, Hq, Hkv, D, B)
    d = to_dev(b)
    log(f"sweep {dt} D={D} B={B} {Hq}/{Hkv}")
    assert_close(gpu_decode(b, d), oracle_decode(b), dt, "sweep")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 4), (16, 2)])
@pytest.mark.parametrize("scale", [-0.09, 0.0, 2.0])
def test_negative_zero_and_large_scales(dtype, Hq, Hkv, scale):
    # groups of 1 (P.V on the vector ALU), 4 and 8 (matrix cores, one reference maximum
    # per head that moves only when a tile exceeds it by 2^8).  A negative scale reverses
    # the score order, 0 gives uniform weights, 2.0 spreads the scores over about +-70 in
    # log2 units so the reference maximum moves often and most weights underflow.
    b = random_batch(400 + Hq + Hkv, dtype, [1, 17, 300, 1031, 64], Hq, Hkv, 128, 16)
    b.scale = scale
    d = to_dev(b)
    log(f"scale {scale} {dtype} {Hq}/{Hkv}")
    assert_close(gpu_decode(b, d), oracle_decode(b), dtype, f"scale {scale}")


@pytest.mark.parametrize("num_seqs", [2048, 2100])
def test_many_sequences_around_the_lds_limit(num_seqs):
    # up to 2048 sequences the decode kernel keeps lengths and tile prefix sums in LDS;
    # beyond that it scans the lengths in global memory.  Short lengths, some empty.
    g = torch.Generator().manual_seed(num_seqs)
    lens = torch.randint(0, 41, (num_seqs,), generator=g)
    lens[torch.randint(0, num_seqs, (64,), generator=g)] = 0
    b = random_batch(300 + num_seqs, "bf16", lens.tolist(), 8, 2, 128, 16)
    d = to_dev(b)
    log(f"{num_seqs} sequences")
    got = gpu_decode(b, d)
    empty = np.where(np.asarray(lens) == 0)[0]
    assert np.array_equal(got[empty], np.zeros_like(got[empty]))
    assert_close(got, oracle_decode(b), "bf16", f"{num_seqs} sequences")


# ---------------------------------------------------------------------------- invariants


def test_deterministic_and_invariant_under_block_relabelling():
    b = random_batch(21, "bf16", [700, 1500, 33, 2048], 32, 8, 128, 16, extra=40)
    d = to_dev(b)
    log("determinism + relabelling")
    o1 = gpu_decode(b, d)
    o2 = gpu_decode(b, d)
    assert np.array_equal(o1, o2)
    g = torch.Generator().manual_seed(5)
    pi = torch.randperm(b.num_blocks, generator=g)
    kc2 = torch.empty_like(b.k_cache)
    vc2 = torch.empty_like(b.v_cache)
    kc2[pi] = b.k_cache
    vc2[pi] = b.v_cache
    bt2 = torch.where(b.block_tables >= 0, pi[b.block_tables.clamp(min=0).long()].int(),
                      b.block_tables)
    d.bt = bt2.cuda()
    o3 = gpu_decode(b, d, kc=kc2.cuda(), vc=vc2.cuda())
    assert np.array_equal(o1, o3)
    assert_close(o1, oracle_decode(b), "bf16", "relabel")


def test_workspace_not_zeroed_before_first_call():
    # The contract asks for a zero-filled workspace before the first call.  One filled
    # with 0xFF bytes instead starts the tail counter at -1: that ticket hands out no
    # chunk, every tail part is still taken once, every access stays in bounds, and the
    # call leaves the counter at 0, so both calls match the oracle.
    rng = np.random.default_rng(29)
    lens = rng.integers(500, 3000, 64).tolist()
    b = random_batch(29, "bf16", lens, 32, 8, 128, 16)
    d = to_dev(b)
    m = pk()
    ws = m.decode_workspace(d.q, b.num_kv_heads, max(lens))
    assert ws is not None
    ws.fill_(255)
    log("decode with a 0xFF-filled workspace, twice")
    ref = oracle_decode(b)
    for call in range(2):
        out = torch.empty_like(d.q)
        m.pa_decode(d.q, d.kc, d.vc, d.bt, d.lens, b.num_kv_heads, b.scale, out,
                    max_seq_len=max(lens), workspace=ws)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().double().numpy(), ref, "bf16", f"0xFF workspace, call {call}")


def test_write_kv_is_bit_exact_on_arbitrary_bit_patterns():
    torch.manual_seed(0)
    NB, B, H, D, T = 50, 16, 8, 128, 300
    kc = torch.randint(-2**15, 2**15, (NB, B, H, D), dtype=torch.int16)
    vc = torch.randint(-2**15, 2**15, (NB, B, H, D), dtype=torch.int16)
    k = torch.randint(-2**15, 2**15, (T, H, D), dtype=torch.int16)
    v = torch.randint(-2**15, 2**15, (T, H, D), dtype=torch.int16)
    slots = torch.randperm(NB * B)[:T].int()
    slots[::7] = -1
    slots[5] = NB * B + 3          # beyond the pool: skipped
    log("write_kv bit patterns")
    dk, dv, ds = k.cuda(), v.cuda(), slots.cuda()
    dkc, dvc = kc.cuda(), vc.cuda()
    pk().pa_write_kv(dk.view(torch.bfloat16), dv.view(torch.bfloat16), ds,
                     dkc.view(torch.bfloat16), dvc.view(torch.bfloat16))
    torch.cuda.synchronize()
    s = slots.numpy().copy()
    s[5] = -1                      # the oracle's contract: in-pool slots only
    ek, ev = oracle.write_kv(k.numpy(), v.numpy(), s, kc.numpy(), vc.numpy())
    assert torch.equal(dkc.cpu(), torch.from_numpy(ek))
    assert torch.equal(dvc.cpu(), torch.from_numpy(ev))


@pytest.mark.parametrize("dtype,H,D,B", [("f16", 40, 128, 16), ("f32", 4, 64, 8), ("bf16", 8, 128, 32)])
def test_copy_blocks_is_bit_exact(dtype, H, D, B):
    torch.manual_seed(1)
    NB = 60
    it = torch.int32 if dtype == "f32" else torch.int16
    lo, hi = (-2**31, 2**31 - 1) if dtype == "f32" else (-2**15, 2**15)
    kc = torch.randint(lo, hi, (NB, B, H, D), dtype=it)
    vc = torch.randint(lo, hi, (NB, B, H, D), dtype=it)
    perm = torch.randperm(NB)
    pairs = torch.stack([perm[:20].repeat_interleave(1), perm[20:40]], 1).int()
    pairs[3, 0] = pairs[2, 0]      # one source copied twice
    log(f"copy_blocks {dtype}")
    dkc, dvc = kc.cuda(), vc.cuda()
    tdt = TORCH_DTYPE[dtype]
    pk().pa_copy_blocks(dkc.view(tdt), dvc.view(tdt), pairs.cuda())
    torch.cuda.synchronize()
    ek, ev = oracle.copy_blocks(kc.numpy(), vc.numpy(), pairs.numpy())
    assert torch.equal(dkc.cpu(), torch.from_numpy(ek))
    assert torch.equal(dvc.cpu(), torch.from_numpy(ev))


# ---------------------------------------------------------------------------- workloads, reduced


@pytest.mark.parametrize("name,make", [
    ("llama7b", lambda: workloads.llama7b(num_seqs=8)),
    ("llama3_8b", lambda: workloads.llama3_8b(num_seqs=16, num_blocks=3000)),
    ("llama2_70b_b8", lambda: workloads.llama2_70b(block_size=8, num_seqs=2)),
    ("llama2_70b_b16", lambda: workloads.llama2_70b(block_size=16, num_seqs=2)),
    ("llama2_70b_b32", lambda: workloads.llama2_70b(block_size=32, num_seqs=2)),
    ("opt13b_shared", lambda: workloads.opt13b_shared(num_prompts=3)),
])
def test_workloads_reduced(name, make):
    b = make()
    d = to_dev(b)
    if b.slot_mapping is not None:
        log(f"{name}: write step")
        pk().pa_write_kv(d.new_k, d.new_v, d.slots, d.kc, d.vc)
        kc2, vc2 = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(b.slot_mapping),
                                   as_numpy(b.k_cache), as_numpy(b.v_cache))
        torch.cuda.synchronize()
        assert torch.equal(bits(d.kc.cpu()), bits(torch.from_numpy(kc2)))
        assert torch.equal(bits(d.vc.cpu()), bits(torch.from_numpy(vc2)))
        b.k_cache, b.v_cache = torch.from_numpy(kc2), torch.from_numpy(vc2)
        if b.dtype == "bf16":
            b.k_cache, b.v_cache = b.k_cache.view(torch.bfloat16), b.v_cache.view(torch.bfloat16)
    log(f"{name}: decode")
    assert_close(gpu_decode(b, d), oracle_decode(b), b.dtype, name)


def test_cow_copy_write_decode_reduced():
    b = workloads.opt13b_cow(num_prompts=3)
    d = to_dev(b)
    m = pk()
    log("opt13b_cow reduced: copy, write, decode")
    m.pa_copy_blocks(d.kc, d.vc, d.pairs)
    m.pa_write_kv(d.new_k, d.new_v, d.slots, d.kc, d.vc)
    kc1, vc1 = oracle.copy_blocks(as_numpy(b.k_cache), as_numpy(b.v_cache), as_numpy(b.cow_pairs))
    kc2, vc2 = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(b.slot_mapping),
                               kc1, vc1)
    got = gpu_decode(b, d)
    assert torch.equal(bits(d.kc.cpu()), bits(torch.from_numpy(kc2)))
    assert torch.equal(bits(d.vc.cpu()), bits(torch.from_numpy(vc2)))
    ref = oracle.paged_decode(as_numpy(b.q), kc2, vc2, as_numpy(b.block_tables),
                              as_numpy(b.seq_lens), b.scale, "f16")
    assert_close(got, ref, "f16", "cow")
    # the 8 samples of a prompt now differ only in their last token
    assert len(b.cow_pairs) == 3 * 7
