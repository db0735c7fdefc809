"""GPU: a decode step captured in a HIP graph and replayed.

A serving loop records its step once and replays it with new inputs copied into the captured
tensors. The step here is pa_write_kv of each sequence's new token followed by pa_decode
(Llama-3-8B shape, reduced batch). The graph is captured through torch's stream capture and
replayed four times with fresh queries and new K/V rows, with unrelated eager work between
replays. The test checks three things:
- Every replay's output and caches equal an eager run of the same step on the same inputs, bit
  for bit. The kernels are deterministic: which wave took which tail chunk never changes a
  result.
- The last replay agrees with the float64 oracle.
- Capture succeeds, which fails on a host synchronisation of the capturing stream. The caller's
  workspace is zeroed once before capture, and the merge kernel leaves it ready for the next
  call, so replays need no memset.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import as_numpy
from _gpu import assert_close, bits, log, pk, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk()


def test_write_and_decode_replayed_from_a_graph():
    m = pk()
    b = workloads.llama3_8b(num_seqs=24, num_blocks=5000)
    d = to_dev(b)
    max_len = int(b.seq_lens.max())
    out_g = torch.empty_like(d.q)
    ws_g = m.decode_workspace(d.q, b.num_kv_heads, max_len)

    def step(q, nk, nv, kc, vc, out, ws):
        m.pa_write_kv(nk, nv, d.slots, kc, vc)
        m.pa_decode(q, kc, vc, d.bt, d.lens, b.num_kv_heads, b.scale, out, max_seq_len=max_len,
                    workspace=ws)

    # eager copies of the caches follow the same writes as the captured ones
    kc_e, vc_e = d.kc.clone(), d.vc.clone()
    ws_e = m.decode_workspace(d.q, b.num_kv_heads, max_len)

    log("graph: warm-up on a side stream, then capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(d.q, d.new_k, d.new_v, d.kc, d.vc, out_g, ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(d.q, d.new_k, d.new_v, d.kc, d.vc, out_g, ws_g)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(77)
    for r in range(4):
        q_r = torch.randn(d.q.shape, generator=gen).to(d.q.dtype)
        nk_r = torch.randn(d.new_k.shape, generator=gen).to(d.new_k.dtype)
        nv_r = torch.randn(d.new_v.shape, generator=gen).to(d.new_v.dtype)
        d.q.copy_(q_r)
        d.new_k.copy_(nk_r)
        d.new_v.copy_(nv_r)
        log(f"graph: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        got = out_g.clone()

        out_e = torch.empty_like(d.q)
        step(q_r.cuda(), nk_r.cuda(), nv_r.cuda(), kc_e, vc_e, out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(out_e)), f"replay {r}: output differs from the eager step"
        assert torch.equal(bits(d.kc), bits(kc_e)) and torch.equal(bits(d.vc), bits(vc_e)), \
            f"replay {r}: caches differ from the eager step"

        # unrelated eager work on the same stream between replays
        x = torch.randn(1 << 20, device="cuda")
        assert torch.isfinite((x * 2).sum())

    log("graph: last replay against the oracle")
    kc2, vc2 = oracle.write_kv(as_numpy(nk_r), as_numpy(nv_r), as_numpy(b.slot_mapping),
                               as_numpy(b.k_cache), as_numpy(b.v_cache))
    seqs = [0, 5, 11, 23]
    ref = oracle.paged_decode(as_numpy(q_r), kc2, vc2, as_numpy(b.block_tables), as_numpy(b.seq_lens),
                              b.scale, b.dtype, seqs=seqs)
    assert_close(got.float().cpu().double().numpy()[seqs], ref, b.dtype, "graph replay")
    assert not np.array_equal(ref, np.zeros_like(ref))
