"""A multi-step decode loop driven by the library's native block manager.

Each step every live sequence reserves the slot of its next token (with
``BlockManager.append_slot`` per sequence on even steps, one
``BlockManager.append_step`` for the batch on odd ones); the copy-on-write pairs of the step go to
``pa_copy_blocks``, the new K/V rows to ``pa_write_kv`` and the batch's block
tables to ``pa_decode``.  Prompts are forked into parallel samples, beams are
pruned and new requests arrive between steps, and the pool is small enough
that the blocks freed by the pruned beams are handed out again.  The check does not use the block manager or
the pool: the test keeps every sequence's K/V history as a dense array (a fork
copies its parent's history) and compares every decode output with the
oracle's plain attention over that history.  Pool slots nobody wrote hold NaN.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.dtypes import to_f64
from workloads import TORCH_DTYPE, as_numpy
from _gpu import assert_close, log, pk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_serving_loop_with_forks_cow_and_reuse(dtype):
    m = pk()
    Hq, Hkv, D, B, NB = 8, 2, 128, 16, 24   # 24 blocks: the loop ends with none free
    tdt = TORCH_DTYPE[dtype]
    g = torch.Generator().manual_seed(351)
    rng = np.random.default_rng(351)
    kc = torch.full((NB, B, Hkv, D), float("nan"), dtype=tdt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    bm = m.BlockManager(NB, B, free_order=rng.permutation(NB).tolist())
    hist = {}                                    # seq -> (K rows, V rows), CPU tensors
    scale = D ** -0.5
    next_id = [0]
    max_blocks = NB

    def rows(n):
        return (torch.randn((n, Hkv, D), generator=g) * 0.5).to(tdt)

    def prefill(n):
        s = next_id[0]
        next_id[0] += 1
        table = bm.allocate(s, n)
        k, v = rows(n), rows(n)
        slots = torch.tensor([table[t // B] * B + t % B for t in range(n)], dtype=torch.int32)
        if n:
            m.pa_write_kv(k.cuda(), v.cuda(), slots.cuda(), kc, vc)
        hist[s] = (k, v)
        return s

    def fork(parent):
        c = next_id[0]
        next_id[0] += 1
        bm.fork(parent, c)
        hist[c] = tuple(t.clone() for t in hist[parent])
        return c

    live = [prefill(n) for n in (37, 16, 1, 70)]
    live += [fork(live[0]) for _ in range(3)] + [fork(live[1])]
    cow_seen = 0
    for step in range(24):
        if step == 6:                            # prune two beams, admit a request
            for s in (live[4], live[1]):
                bm.free_seq(s)
                live.remove(s)
                del hist[s]
            live.append(prefill(29))
        if step == 12:
            live += [fork(live[-1]), fork(live[2])]
        if step % 2:                             # one call for the whole step
            slots, pairs = bm.append_step(live)
            slots, pairs = slots.tolist(), pairs.tolist()
        else:                                    # one call per sequence
            pairs, slots = [], []
            for s in live:
                slot, cow = bm.append_slot(s)
                slots.append(slot)
                if cow is not None:
                    pairs.append(cow)
        cow_seen += len(pairs)
        k, v = rows(len(live)), rows(len(live))
        for i, s in enumerate(live):
            hist[s] = (torch.cat([hist[s][0], k[i:i + 1]]), torch.cat([hist[s][1], v[i:i + 1]]))
        log(f"serving loop {dtype} step {step}: {len(live)} seqs, {len(pairs)} copies, "
            f"{bm.num_free()} free")
        if pairs:
            m.pa_copy_blocks(kc, vc, torch.tensor(pairs, dtype=torch.int32).cuda())
        m.pa_write_kv(k.cuda(), v.cuda(), torch.tensor(slots, dtype=torch.int32).cuda(), kc, vc)
        tables, lens = bm.batch(live, max_blocks)
        q = (torch.randn((len(live), Hq, D), generator=g) * 0.5).to(tdt)
        out = torch.empty((len(live), Hq, D), dtype=tdt, device="cuda")
        m.pa_decode(q.cuda(), kc, vc, tables.cuda(), lens.cuda(), Hkv, scale, out,
                    max_seq_len=int(lens.max()))
        torch.cuda.synchronize()
        got = out.float().cpu().double().numpy()
        ref = np.stack([oracle.attend(to_f64(as_numpy(q[i]), dtype), to_f64(as_numpy(hist[s][0]), dtype),
                                      to_f64(as_numpy(hist[s][1]), dtype), scale)
                        for i, s in enumerate(live)])
        assert_close(got, ref, dtype, f"step {step}")
    assert cow_seen > 0 and bm.num_free() == 0
