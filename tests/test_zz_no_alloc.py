"""pa_decode_no_alloc, the decode entry point that allocates nothing (its workspace is an
array built into the library), through the C ABI: bit-identical to pa_decode with a
caller-owned workspace on the same inputs, on two calls in a row with the second one
smaller, and within tolerance of the float64 oracle."""

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


def _batch(seed, dtype, lens, Hq, Hkv, D, B):
    g = torch.Generator().manual_seed(seed)
    return workloads._paged(name=f"noalloc{seed}", dtype=dtype, lens=lens, Hq=Hq, Hkv=Hkv, D=D, B=B,
                            num_blocks=sum(-(-L // B) for L in lens) + 7, gen=g)


def _both(b):
    """(pa_decode output, pa_decode_no_alloc output) as raw bits and float64."""
    m = pk()
    d = to_dev(b)
    max_len = int(b.seq_lens.max())
    ref = torch.empty_like(d.q)
    m.pa_decode(d.q, d.kc, d.vc, d.bt, d.lens, b.num_kv_heads, b.scale, ref, max_seq_len=max_len)
    got = torch.full_like(d.q, float("nan"))
    m.pa_decode_no_alloc(d.q, d.kc, d.vc, d.bt, d.lens, b.num_kv_heads, b.scale, got,
                         max_seq_len=max_len)
    torch.cuda.synchronize()
    return ref, got


def _same_bits(a, b):
    view = torch.int16 if a.element_size() == 2 else torch.int32
    return torch.equal(a.view(view), b.view(view))


def test_two_calls_second_smaller_match_pa_decode():
    # a large batch (many split pairs, every wave busy), then a small one on the same array
    big = _batch(901, "bf16", [int(x) for x in np.random.default_rng(5).integers(512, 4097, 192)],
                 32, 8, 128, 16)
    small = _batch(902, "bf16", [1, 7, 16, 40, 300, 1031], 32, 8, 128, 16)
    for what, b in (("first call, 192 sequences", big), ("second call, 6 sequences", small)):
        log(f"no-alloc: {what}")
        ref, got = _both(b)
        assert _same_bits(ref, got), what
        seqs = list(range(min(6, b.num_seqs)))
        assert_close(got.float().cpu().double().numpy()[seqs], oracle_decode(b, seqs=seqs), "bf16", what)


@pytest.mark.parametrize("dtype,Hq,Hkv,D,B", [("f32", 4, 4, 64, 16), ("f16", 40, 40, 128, 16),
                                              ("bf16", 64, 8, 128, 32)])
def test_other_shapes_match_pa_decode(dtype, Hq, Hkv, D, B):
    b = _batch(903, dtype, [0, 1, 17, 250, 2049, 33], Hq, Hkv, D, B)
    log(f"no-alloc: {dtype} {Hq}/{Hkv} D={D} B={B}")
    ref, got = _both(b)
    assert _same_bits(ref, got)
    assert_close(got.float().cpu().double().numpy(), oracle_decode(b), dtype, "no-alloc")


def test_scratch_size_is_reported():
    assert pk().pa_decode_no_alloc_scratch_bytes() == 34 << 20
