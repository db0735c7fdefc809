"""The binding on a stream other than the current one, with no workspace passed: the
binding allocates (and, for pa_decode, zero-fills) the workspace on the stream the call
runs on, so the fill is ordered before the kernels even while the current stream is busy,
and the memory is not handed to another stream's work while the call may still use it.

Each call is preceded by work on the current stream (a chain of matrix products) and by a
workspace-sized block filled with 0xFF on the side stream and freed, which the caching
allocator hands back next: a fill left on the busy current stream would leave that 0xFF
in place when the kernels start."""

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


def _busy_current_stream():
    a = torch.randn(4096, 4096, device="cuda")
    for _ in range(8):
        a = a @ a
        a = a / a.abs().max()
    return a


def _poison(nbytes, side):
    with torch.cuda.stream(side):
        t = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    del t


def test_pa_decode_on_a_side_stream_without_workspace():
    m = pk()
    side = torch.cuda.Stream()
    for seed, lens in ((31, [700, 1, 33, 4096, 2000, 15]), (32, [513, 9, 3000])):
        g = torch.Generator().manual_seed(seed)
        b = workloads._paged(name=f"side{seed}", dtype="bf16", lens=lens, Hq=32, Hkv=8, D=128, B=16,
                             gen=g)
        d = to_dev(b)
        torch.cuda.synchronize()
        max_len = max(lens)
        _poison(m.pa_decode_workspace_size(b.num_seqs, 32, 8, 128, max_len), side)
        keep = _busy_current_stream()
        out = torch.empty_like(d.q)
        side.wait_stream(torch.cuda.current_stream())     # inputs were made on the current stream
        log(f"side stream pa_decode, lens {lens}")
        m.pa_decode(d.q, d.kc, d.vc, d.bt, d.lens, 8, b.scale, out, max_seq_len=max_len, stream=side)
        torch.cuda.synchronize()
        del keep
        assert_close(out.float().cpu().double().numpy(), oracle_decode(b), "bf16", "side stream")


def test_pa_multi_query_on_a_side_stream_without_workspace():
    m = pk()
    side = torch.cuda.Stream()
    b = workloads.multi_query_small(seed=33, dtype="bf16", lens=(300, 40, 1200, 64),
                                    queries=(3, 40, 2, 64), Hq=32, Hkv=8, D=128, B=16)
    d = to_dev(b)
    qs = b.q_start.cuda()
    m.pa_write_kv(d.new_k, d.new_v, d.slots, d.kc, d.vc)
    torch.cuda.synchronize()
    need = m.pa_multi_query_workspace_size(b.num_seqs, b.q.shape[0], 32, 8, 128, b.max_q_len,
                                           b.max_seq_len)
    _poison(max(need, 256), side)
    keep = _busy_current_stream()
    out = torch.empty_like(d.q)
    side.wait_stream(torch.cuda.current_stream())
    log("side stream pa_multi_query")
    m.pa_multi_query(d.q, d.kc, d.vc, d.bt, d.lens, qs, 8, b.scale, out, max_q_len=b.max_q_len,
                     max_seq_len=b.max_seq_len, stream=side)
    torch.cuda.synchronize()
    del keep
    import oracle
    from workloads import as_numpy
    kc, vc = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(b.slot_mapping),
                             as_numpy(b.k_cache), as_numpy(b.v_cache))
    ref = oracle.paged_multi_query(as_numpy(b.q), kc, vc, as_numpy(b.block_tables), as_numpy(b.seq_lens),
                                   as_numpy(b.q_start), b.scale, "bf16")
    assert_close(out.float().cpu().double().numpy(), ref, "bf16", "side stream multi-query")
