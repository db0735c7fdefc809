"""GPU: pa_swap_blocks (preemption, [PA-notes] §5 ③) and a decode loop that swaps.

Swaps move bits, so they must match ``oracle.swap_blocks`` bit for bit over the
whole destination pool, for GPU -> pinned host, pinned host -> GPU and GPU ->
GPU, with the pair list on the device or in pinned host memory.  Pageable host
memory must be refused before anything is launched.  The loop test preempts a
group of samples (swap-out), keeps decoding the others while the freed blocks
are reused, restores the group (swap-in, into different blocks) and checks
every decode against the oracle's attention over per-sequence histories.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from oracle.dtypes import to_f64
from workloads import TORCH_DTYPE, as_numpy
from _gpu import assert_close, bits, log, pk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk()


def random_bits(shape, dtype, g):
    n = int(np.prod(shape))
    if dtype == torch.float32:
        raw = torch.randint(-2**31, 2**31 - 1, (n,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        raw = torch.randint(-2**15, 2**15 - 1, (n,), generator=g, dtype=torch.int64).to(torch.int16)
    return raw.view(dtype).reshape(shape)


@pytest.mark.parametrize("direction", ["out", "in", "d2d"])
@pytest.mark.parametrize("pairs_on", ["device", "pinned"])
@pytest.mark.parametrize("dtype,H,D,B", [(torch.bfloat16, 8, 128, 16), (torch.float16, 2, 64, 32),
                                         (torch.float32, 1, 64, 1)])
def test_swap_is_bit_exact(direction, pairs_on, dtype, H, D, B):
    m = pk()
    g = torch.Generator().manual_seed(7)
    NG, NC = 37, 23
    gk, gv = random_bits((NG, B, H, D), dtype, g), random_bits((NG, B, H, D), dtype, g)
    ck, cv = random_bits((NC, B, H, D), dtype, g), random_bits((NC, B, H, D), dtype, g)
    if direction == "out":
        src, dst = (gk.cuda(), gv.cuda()), (ck.pin_memory(), cv.pin_memory())
        ns, nd = NG, NC
    elif direction == "in":
        src, dst = (ck.pin_memory(), cv.pin_memory()), (gk.cuda(), gv.cuda())
        ns, nd = NC, NG
    else:
        src, dst = (gk.cuda(), gv.cuda()), (ck.cuda(), cv.cuda())
        ns, nd = NG, NC
    rng = np.random.default_rng(1)
    n = min(ns, nd) - 3
    pairs = np.stack([rng.choice(ns, n, replace=False), rng.choice(nd, n, replace=False)], 1)
    pt = torch.from_numpy(pairs.astype(np.int32))
    pt = pt.cuda() if pairs_on == "device" else pt.pin_memory()
    src_np = [as_numpy(t.cpu()) for t in src]
    dst_np = [as_numpy(t.cpu()) for t in dst]
    log(f"swap {direction} pairs={pairs_on} {dtype} H={H} D={D} B={B}: {n} blocks")
    m.pa_swap_blocks(src[0], src[1], dst[0], dst[1], pt)
    torch.cuda.synchronize()
    ek, ev = oracle.swap_blocks(src_np[0], src_np[1], dst_np[0], dst_np[1], pairs)
    for got, exp in ((dst[0], ek), (dst[1], ev)):
        assert torch.equal(bits(got.cpu()), bits(torch.from_numpy(exp).view(got.dtype)
                                                 if exp.dtype == np.uint16 else torch.from_numpy(exp)))
    # the sources are untouched
    for t, ref in zip(src, src_np):
        assert np.array_equal(as_numpy(t.cpu()).view(np.uint8), ref.view(np.uint8))


def test_pageable_host_memory_is_refused():
    m = pk()
    L = m.lib()
    gk = torch.zeros((4, 16, 2, 64), dtype=torch.float16, device="cuda")
    host = torch.zeros((4, 16, 2, 64), dtype=torch.float16)      # pageable
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    log("swap refuses pageable memory")
    st = L.pa_swap_blocks(ctypes.c_void_p(gk.data_ptr()), ctypes.c_void_p(gk.data_ptr()), 4,
                          ctypes.c_void_p(host.data_ptr()), ctypes.c_void_p(host.data_ptr() + 0), 4,
                          ctypes.c_void_p(pairs.data_ptr()), 1, 16, 2, 64, 1, None)
    assert st == 1 and "pinned" in m.pa_last_error()
    with pytest.raises(ValueError):
        m.pa_swap_blocks(gk, gk, host, host, pairs)
    # the runtime is still healthy afterwards
    torch.cuda.synchronize()
    assert float(gk.sum()) == 0.0


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_loop_with_preemption(dtype):
    m = pk()
    Hq, Hkv, D, B, NB, NC = 8, 2, 128, 16, 17, 20   # 17 blocks: the pool ends full
    tdt = TORCH_DTYPE[dtype]
    g = torch.Generator().manual_seed(5)
    rng = np.random.default_rng(5)
    kc = torch.full((NB, B, Hkv, D), float("nan"), dtype=tdt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    hk = torch.full((NC, B, Hkv, D), float("nan"), dtype=tdt).pin_memory()
    hv = torch.full((NC, B, Hkv, D), float("nan"), dtype=tdt).pin_memory()
    bm = m.BlockManager(NB, B, free_order=rng.permutation(NB).tolist(), num_cpu_blocks=NC)
    hist, scale, next_id = {}, D ** -0.5, [0]

    def rows(n):
        return (torch.randn((n, Hkv, D), generator=g) * 0.5).to(tdt)

    def prefill(n):
        s = next_id[0]
        next_id[0] += 1
        table = bm.allocate(s, n)
        k, v = rows(n), rows(n)
        slots = torch.tensor([table[t // B] * B + t % B for t in range(n)], dtype=torch.int32)
        m.pa_write_kv(k.cuda(), v.cuda(), slots.cuda(), kc, vc)
        hist[s] = (k, v)
        return s

    def fork(p):
        c = next_id[0]
        next_id[0] += 1
        bm.fork(p, c)
        hist[c] = tuple(t.clone() for t in hist[p])
        return c

    prompt = prefill(45)                          # 3 blocks, last one partly filled
    group = [prompt] + [fork(prompt) for _ in range(3)]
    for n in (20, 33):
        prefill(n)
    swaps = 0
    for step in range(16):
        if step == 3:                             # preempt the sample group
            pairs = bm.swap_out(group)
            log(f"{dtype} step {step}: swap out {len(pairs)} blocks")
            m.pa_swap_blocks(kc, vc, hk, hv, pairs.cuda())
            swaps += len(pairs)
            freed = set(pairs[:, 0].tolist())
            for s in group:
                assert bm.is_swapped(s)
        if step == 4:                             # a long newcomer overwrites freed blocks
            newcomer = prefill(150)
            assert set(bm.table(newcomer)) & freed
        if step == 8:                             # ... and finishes
            bm.free_seq(newcomer)
            del hist[newcomer]
        if step == 9:                             # restore the group into fresh blocks
            pairs = bm.swap_in(group)
            log(f"{dtype} step {step}: swap in {len(pairs)} blocks")
            m.pa_swap_blocks(hk, hv, kc, vc, pairs.pin_memory())
            swaps += len(pairs)
        live = [s for s in list(hist) if not bm.is_swapped(s)]
        slots, pairs = bm.append_step(live)
        if len(pairs):
            m.pa_copy_blocks(kc, vc, pairs.cuda())
        k, v = rows(len(live)), rows(len(live))
        for i, s in enumerate(live):
            hist[s] = (torch.cat([hist[s][0], k[i:i + 1]]), torch.cat([hist[s][1], v[i:i + 1]]))
        m.pa_write_kv(k.cuda(), v.cuda(), slots.cuda(), kc, vc)
        tables, lens = bm.batch(live, NB)
        q = (torch.randn((len(live), Hq, D), generator=g) * 0.5).to(tdt)
        out = torch.empty((len(live), Hq, D), dtype=tdt, device="cuda")
        m.pa_decode(q.cuda(), kc, vc, tables.cuda(), lens.cuda(), Hkv, scale, out,
                    max_seq_len=int(lens.max()))
        torch.cuda.synchronize()
        ref = np.stack([oracle.attend(to_f64(as_numpy(q[i]), dtype), to_f64(as_numpy(hist[s][0]), dtype),
                                      to_f64(as_numpy(hist[s][1]), dtype), scale)
                        for i, s in enumerate(live)])
        assert_close(out.float().cpu().double().numpy(), ref, dtype, f"step {step}")
    assert swaps > 0 and bm.num_free_cpu() == NC and bm.num_free() == 0
