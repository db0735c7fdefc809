"""pa_decode_cached: pa_decode with the default cache policy for its K/V loads, for batches
whose sequences share blocks ([PA-notes] "LLM 注意力与计算内核精读笔记 · 05 PagedAttention 与
KV 显存管理" §6.1 parallel sampling, §6.2 beam search).  Only the cache hint differs from
pa_decode, so the outputs must be equal bit for bit; one shared-block batch is also held to
the oracle's tolerance."""

import numpy as np
import pytest
import torch

import workloads
from _gpu import assert_close, log, oracle_decode, pk, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk()


def bits(t):
    t = t.contiguous().cpu()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def both(b):
    m = pk()
    d = to_dev(b)
    if d.pairs is not None:
        m.pa_copy_blocks(d.kc, d.vc, d.pairs)
    if d.slots is not None:
        m.pa_write_kv(d.new_k, d.new_v, d.slots, d.kc, d.vc)
    outs = []
    for fn in (m.pa_decode, m.pa_decode_cached):
        out = torch.full_like(d.q, 7.0)
        fn(d.q, d.kc, d.vc, d.bt, d.lens, b.num_kv_heads, b.scale, out, max_seq_len=b.max_seq_len)
        outs.append(out)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("make", [
    lambda: workloads.tiny(),
    lambda: workloads.llama3_8b(num_seqs=24, max_len=1500, num_blocks=3000),
    lambda: workloads.llama2_70b(block_size=8, num_seqs=3, min_len=3000, max_len=5000),
    lambda: workloads.llama7b(num_seqs=10, max_len=700),
    lambda: workloads.opt13b_shared(num_prompts=3, samples=4, prompt_len=192, tail_max=40),
], ids=["tiny", "llama3_8b_small", "llama2_70b_b8_small", "llama7b_small", "opt13b_shared_small"])
def test_same_bits_as_pa_decode(make):
    b = make()
    a, c = both(b)
    assert np.array_equal(bits(a), bits(c)), f"{b.name}: pa_decode_cached differs from pa_decode"
    log(f"decode_cached {b.name}: bit-identical to pa_decode")


def test_shared_blocks_against_oracle():
    b = workloads.opt13b_cow(num_prompts=2, samples=4, prompt_len=200)
    _, c = both(b)
    import oracle
    from workloads import as_numpy
    kc, vc = as_numpy(b.k_cache), as_numpy(b.v_cache)
    if b.cow_pairs is not None:
        kc, vc = oracle.copy_blocks(kc, vc, as_numpy(b.cow_pairs))
    if b.slot_mapping is not None:
        kc, vc = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(b.slot_mapping), kc, vc)
    ref = oracle.paged_decode(as_numpy(b.q), kc, vc, as_numpy(b.block_tables), as_numpy(b.seq_lens),
                              b.scale, b.dtype)
    assert_close(c.float().cpu().double().numpy(), ref, b.dtype, "opt13b_cow small, pa_decode_cached")
    log("decode_cached opt13b_cow small: within tolerance of the oracle")
