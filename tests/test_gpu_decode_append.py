"""pa_decode_append: each sequence's newest token (position L - 1) stored into the slot its
block table gives that position, then the decode, in one call ([PA-notes] "LLM 注意力与计算
内核精读笔记 · 05 PagedAttention 与 KV 显存管理" §5 ② for the append into the last block's
next slot, §4 for the decode).

Every case runs the two-call path (pa_write_kv into those slots, then pa_decode) on one copy
of the pool and pa_decode_append on another: the outputs and both whole pools must be equal
bit for bit.  The fused output is also held to the dtype tolerance of the float64 oracle's
write followed by its decode, on every sequence."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from _gpu import assert_close, log, pk
from workloads import as_numpy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk()


def bits(t):
    t = t.contiguous().cpu()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def newest_slots(b, lens):
    """Slot of position L - 1 of every sequence (-1 for an empty one), from the tables."""
    bt = b.block_tables
    B = b.block_size
    out = []
    for s, L in enumerate(lens.tolist()):
        out.append(int(bt[s, (L - 1) // B]) * B + (L - 1) % B if L > 0 else -1)
    return torch.tensor(out, dtype=torch.int32)


def run_both(b, lens=None, dev="cuda"):
    """Two-call path and fused call on copies of the same pool; returns (outputs, pools)."""
    m = pk()
    lens = b.seq_lens if lens is None else lens
    max_len = int(lens.max()) if lens.numel() else 0
    q, bt, ld = b.q.to(dev), b.block_tables.to(dev), lens.to(dev)
    nk, nv = b.new_k.to(dev), b.new_v.to(dev)
    slots = newest_slots(b, lens)
    if b.slot_mapping is not None:
        live = lens > 0
        assert torch.equal(slots[live], b.slot_mapping[live]), "workload's write slots are not the newest"
    res = {}
    for how in ("two_calls", "fused"):
        kc, vc = b.k_cache.to(dev), b.v_cache.to(dev)
        out = torch.full_like(q, 7.0)
        if how == "two_calls":
            m.pa_write_kv(nk, nv, slots.to(dev), kc, vc)
            m.pa_decode(q, kc, vc, bt, ld, b.num_kv_heads, b.scale, out, max_seq_len=max_len)
        else:
            m.pa_decode_append(q, nk, nv, kc, vc, bt, ld, b.num_kv_heads, b.scale, out,
                               max_seq_len=max_len)
        torch.cuda.synchronize()
        res[how] = (out, kc, vc)
    return res, slots


def check_case(b, lens=None, what="", oracle_check=True):
    lens = b.seq_lens if lens is None else lens
    res, slots = run_both(b, lens)
    (oa, ka, va), (ob, kb, vb) = res["two_calls"], res["fused"]
    assert np.array_equal(bits(oa), bits(ob)), f"{what}: output bits differ from write + decode"
    assert np.array_equal(bits(ka), bits(kb)), f"{what}: K pool differs from write + decode"
    assert np.array_equal(bits(va), bits(vb)), f"{what}: V pool differs from write + decode"
    if oracle_check:
        kc, vc = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(slots),
                                 as_numpy(b.k_cache), as_numpy(b.v_cache))
        ref = oracle.paged_decode(as_numpy(b.q), kc, vc, as_numpy(b.block_tables), as_numpy(lens),
                                  b.scale, b.dtype)
        assert_close(ob.float().cpu().double().numpy(), ref, b.dtype, what)
    log(f"decode_append {what}: bit-identical to write + decode"
        + (", oracle within tolerance" if oracle_check else ""))


def paged(dtype, lens, Hq, Hkv, D, B, seed, num_blocks=None):
    g = torch.Generator().manual_seed(seed)
    return workloads._paged(name=f"append_{dtype}", dtype=dtype, lens=lens, Hq=Hq, Hkv=Hkv, D=D, B=B,
                            num_blocks=num_blocks, gen=g, write_last=True)


def test_tiny():
    check_case(workloads.tiny(seed=0), what="tiny (f32, 4 sequences, 2/8/17/41 tokens)")


def test_worked_example_block_9():
    # the 40-token request on blocks 5, 2, 9 plus the appended token at position 40 (block 9)
    for dtype in ("f32", "f16", "bf16"):
        check_case(workloads.worked_5_2_9(dtype=dtype), what=f"blocks 5, 2, 9 ({dtype})")


# newest tokens at every place in a tile and a block: first and last slot of a block, first
# and last token of a 16-token tile, single-token sequences
EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 49, 64, 65, 100, 129, 257]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,B", [
    ("bf16", 32, 8, 128, 16),    # matrix-core P.V, the Llama-3-8B group
    ("bf16", 8, 8, 128, 16),     # group 1: vector-ALU P.V
    ("f16", 16, 2, 64, 8),       # group 8, two blocks per tile
    ("f16", 4, 2, 128, 32),      # group 2, two tiles per block
    ("f32", 12, 4, 64, 16),      # group 3 (padded to 4)
    ("f32", 16, 1, 128, 8),      # group 16
    ("bf16", 8, 2, 64, 32),
])
def test_edge_lengths(dtype, Hq, Hkv, D, B):
    b = paged(dtype, EDGE_LENS, Hq, Hkv, D, B, seed=11 + Hq + D + B)
    check_case(b, what=f"{dtype} Hq={Hq} Hkv={Hkv} D={D} B={B}, lengths {EDGE_LENS}")


def test_split_pairs():
    # three long sequences, two KV heads: six pairs cut over about a thousand waves, so the
    # newest token's tile sits in a tail chunk or a later piece of a split pair
    b = paged("bf16", [3001, 4096, 5000], 8, 2, 128, 16, seed=5)
    check_case(b, what="bf16, 3 sequences of 3001/4096/5000 tokens (split pairs)")
    b = paged("f16", [777, 2049], 32, 4, 64, 8, seed=6)
    check_case(b, what="f16 B=8, 2 sequences of 777/2049 tokens (split pairs)")


def test_empty_sequences_append_nothing():
    b = paged("bf16", [40, 17, 300, 5, 64], 8, 2, 128, 16, seed=8)
    lens = b.seq_lens.clone()
    lens[1] = 0
    lens[3] = 0
    check_case(b, lens=lens, what="bf16 with two empty sequences (their rows unused)")


def test_repeated_calls_are_idempotent():
    # a serving loop that retries a step: the second call finds its slots already written
    m = pk()
    b = paged("bf16", [33, 500, 1000, 7], 32, 8, 128, 16, seed=9)
    dev = "cuda"
    q, bt, ld = b.q.to(dev), b.block_tables.to(dev), b.seq_lens.to(dev)
    nk, nv = b.new_k.to(dev), b.new_v.to(dev)
    kc, vc = b.k_cache.to(dev), b.v_cache.to(dev)
    ws = m.decode_workspace(q, b.num_kv_heads, b.max_seq_len)
    outs = []
    for _ in range(3):
        out = torch.empty_like(q)
        m.pa_decode_append(q, nk, nv, kc, vc, bt, ld, b.num_kv_heads, b.scale, out,
                           max_seq_len=b.max_seq_len, workspace=ws)
        outs.append(bits(out))
    torch.cuda.synchronize()
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    log("decode_append: three calls on one workspace give the same bits")


def test_llama3_8b_full_size():
    # the benchmark's layer: 256 sequences, 32/8 heads, bf16, 70,000-block pool; bits against
    # write + decode on every sequence and both whole pools, the oracle on every sequence
    b = workloads.llama3_8b(seed=0)
    check_case(b, what="Llama-3-8B shape, 256 sequences (full size)")
