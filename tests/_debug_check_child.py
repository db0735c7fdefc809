"""Child process of tests/test_gpu_debug_check.py, started with PA_DEBUG_CHECK=1 in its
environment before anything touches the GPU.

It hands every entry point index data that breaks the contract of include/pagedkv.h
(block ids outside the pool, slots outside the pool or named twice, newest slots that
are shared, copy pairs that
overlap, swap pairs with a repeated destination, bad q_start / group_start /
prefix_lens) and records, per case, the status, the message and whether the output or
the pool was left untouched (a rejected call must launch nothing).  Then it runs the
valid inputs of every entry point and saves their outputs, which the parent compares
bit for bit with a run without the debug checks.

    python tests/_debug_check_child.py OUT_DIR      (prints one JSON line)
"""

import json
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import paged_kv_cache_351_amd as pk  # noqa: E402
import workloads  # noqa: E402


def inputs():
    """The seeded inputs both processes use (CPU tensors)."""
    g = torch.Generator().manual_seed(77)
    dec = workloads._paged(name="dbg_decode", dtype="bf16", lens=[1, 17, 40, 300], Hq=8, Hkv=2,
                           D=128, B=16, num_blocks=40, gen=g, write_last=True)
    mq = workloads.multi_query_small(seed=78, dtype="f16")
    sh = workloads._shared(name="dbg_shared", seed=79, num_prompts=2, samples=3, prompt_len=48,
                           tail_max=20, cow=False, Hq=4, D=64, B=16, fill="nan")
    return dec, mq, sh


def bits(t):
    t = t.contiguous().cpu()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def run_valid(dec, mq, sh, dev="cuda"):
    """Every entry point on valid inputs; returns their outputs (and the written pool) as
    raw bits."""
    out = {}
    q, kc, vc = dec.q.to(dev), dec.k_cache.to(dev), dec.v_cache.to(dev)
    bt, lens = dec.block_tables.to(dev), dec.seq_lens.to(dev)
    pk.pa_write_kv(dec.new_k.to(dev), dec.new_v.to(dev), dec.slot_mapping.to(dev), kc, vc)
    free = [b for b in range(dec.num_blocks) if b not in set(dec.block_tables[dec.block_tables >= 0].tolist())]
    pairs = torch.tensor([[int(dec.block_tables[3, 0]), free[0]], [int(dec.block_tables[2, 1]), free[1]]],
                         dtype=torch.int32, device=dev)
    pk.pa_copy_blocks(kc, vc, pairs)
    o = torch.empty_like(q)
    pk.pa_decode(q, kc, vc, bt, lens, dec.num_kv_heads, dec.scale, o, max_seq_len=300)
    out["decode"] = bits(o)
    o2 = torch.empty_like(q)
    pk.pa_decode_no_alloc(q, kc, vc, bt, lens, dec.num_kv_heads, dec.scale, o2, max_seq_len=300)
    out["decode_no_alloc"] = bits(o2)
    out["pool_k"], out["pool_v"] = bits(kc), bits(vc)
    hk = torch.zeros((8,) + tuple(kc.shape[1:]), dtype=kc.dtype).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    pk.pa_swap_blocks(kc, vc, hk, hv, torch.tensor([[free[0], 3], [int(dec.block_tables[0, 0]), 5]],
                                                   dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    out["swap_k"], out["swap_v"] = bits(hk), bits(hv)
    mo = torch.empty(mq.q.shape, dtype=mq.q.dtype, device=dev)
    pk.pa_multi_query(mq.q.to(dev), mq.k_cache.to(dev), mq.v_cache.to(dev), mq.block_tables.to(dev),
                      mq.seq_lens.to(dev), mq.q_start.to(dev), mq.num_kv_heads, mq.scale, mo,
                      max_q_len=mq.max_q_len, max_seq_len=mq.max_seq_len)
    out["multi_query"] = bits(mo)
    so = torch.empty(sh.q.shape, dtype=sh.q.dtype, device=dev)
    pk.pa_decode_shared_prefix(sh.q.to(dev), sh.k_cache.to(dev), sh.v_cache.to(dev),
                               sh.block_tables.to(dev), sh.seq_lens.to(dev), sh.group_start.to(dev),
                               sh.prefix_lens.to(dev), sh.num_kv_heads, sh.scale, so, max_group_size=3,
                               max_seq_len=sh.max_seq_len)
    out["shared_prefix"] = bits(so)
    ak, av = dec.k_cache.to(dev), dec.v_cache.to(dev)
    ao = torch.empty_like(q)
    pk.pa_decode_append(q, dec.new_k.to(dev), dec.new_v.to(dev), ak, av, bt, lens, dec.num_kv_heads,
                        dec.scale, ao, max_seq_len=300)
    out["decode_append"] = bits(ao)
    out["append_pool_k"], out["append_pool_v"] = bits(ak), bits(av)
    torch.cuda.synchronize()
    return out


def main():
    assert os.environ.get("PA_DEBUG_CHECK") == "1", "start this process with PA_DEBUG_CHECK=1"
    out_dir = sys.argv[1]
    dev = "cuda"
    pk.lib()
    dec, mq, sh = inputs()
    results = []

    def expect_invalid(name, call, watched):
        """Run a call that breaks the contract; record its status and message and whether
        every watched tensor kept its bits (nothing was launched)."""
        before = [bits(t) for t in watched]
        status, msg = 0, ""
        try:
            call()
        except pk.PagedKVError as e:
            status, msg = e.status, pk.pa_last_error()
        torch.cuda.synchronize()
        same = all(np.array_equal(a, bits(t)) for a, t in zip(before, watched))
        results.append({"case": name, "status": status, "message": msg, "untouched": same})

    # ---- pa_decode and pa_decode_no_alloc: block ids outside the pool, a length above the bound
    q, kc, vc = dec.q.to(dev), dec.k_cache.to(dev), dec.v_cache.to(dev)
    lens = dec.seq_lens.to(dev)
    o = torch.full_like(q, 7.0)
    for name, bad in (("decode table id = num_blocks", dec.num_blocks), ("decode table id = -1", -1)):
        bt = dec.block_tables.clone()
        bt[3, 5] = bad                                  # a block sequence 3 (300 tokens) uses
        btd = bt.to(dev)
        expect_invalid(name, lambda: pk.pa_decode(q, kc, vc, btd, lens, 2, dec.scale, o, max_seq_len=300), [o])
        expect_invalid(name.replace("decode", "decode_no_alloc"),
                       lambda: pk.pa_decode_no_alloc(q, kc, vc, btd, lens, 2, dec.scale, o, max_seq_len=300), [o])
    bt = dec.block_tables.to(dev)
    expect_invalid("decode seq_len above max_seq_len",
                   lambda: pk.pa_decode(q, kc, vc, bt, lens, 2, dec.scale, o, max_seq_len=299), [o])

    # ---- pa_decode_append: two sequences appending into one slot, a newest slot that
    # another sequence reads (sequence 0 appends at position 0 of its block 0, sequence 1
    # at position 16 = offset 0 of its block 1; sequence 2 at position 39 = offset 7 of its
    # block 2, which sequence 3 then also maps as its block 0)
    nk, nv = dec.new_k.to(dev), dec.new_v.to(dev)
    bt = dec.block_tables.clone()
    bt[1, 1] = bt[0, 0]
    btd = bt.to(dev)
    expect_invalid("decode_append two sequences append into one slot",
                   lambda: pk.pa_decode_append(q, nk, nv, kc, vc, btd, lens, 2, dec.scale, o,
                                               max_seq_len=300), [o, kc, vc])
    bt = dec.block_tables.clone()
    bt[3, 0] = bt[2, 2]
    btd2 = bt.to(dev)
    expect_invalid("decode_append newest slot read by another sequence",
                   lambda: pk.pa_decode_append(q, nk, nv, kc, vc, btd2, lens, 2, dec.scale, o,
                                               max_seq_len=300), [o, kc, vc])

    # ---- pa_write_kv: a slot outside the pool, a slot named twice
    nk, nv = dec.new_k.to(dev), dec.new_v.to(dev)
    for name, slots in (("write slot outside the pool", [5, 6, 7, dec.num_blocks * 16]),
                        ("write slot named twice", [5, 6, 6, 9])):
        sl = torch.tensor(slots, dtype=torch.int32, device=dev)
        expect_invalid(name, lambda: pk.pa_write_kv(nk, nv, sl, kc, vc), [kc, vc])

    # ---- pa_copy_blocks: src == dst, a repeated dst, a dst that is also a src, outside the pool
    for name, pairs in (("copy src == dst", [[1, 1]]),
                        ("copy dst repeated", [[1, 2], [3, 2]]),
                        ("copy dst is also a src", [[1, 2], [2, 4]]),
                        ("copy pair outside the pool", [[1, dec.num_blocks]])):
        pr = torch.tensor(pairs, dtype=torch.int32, device=dev)
        expect_invalid(name, lambda: pk.pa_copy_blocks(kc, vc, pr), [kc, vc])

    # ---- pa_swap_blocks: a repeated dst, a pair outside the destination pool
    hk = torch.zeros((8,) + tuple(kc.shape[1:]), dtype=kc.dtype).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    for name, pairs in (("swap dst repeated", [[1, 3], [2, 3]]), ("swap pair outside the pools", [[1, 8]])):
        pr = torch.tensor(pairs, dtype=torch.int32, device=dev)
        expect_invalid(name, lambda: pk.pa_swap_blocks(kc, vc, hk, hv, pr), [hk, hv])

    # ---- pa_multi_query: q_start not from 0 to total_q, too many queries, more queries than
    # tokens, a block id outside the pool
    mqd = [t.to(dev) for t in (mq.q, mq.k_cache, mq.v_cache, mq.block_tables, mq.seq_lens)]
    mo = torch.full(mq.q.shape, 7.0, dtype=mq.q.dtype, device=dev)

    def mq_call(q_start, lens_=None, table=None, max_q_len=None):
        return lambda: pk.pa_multi_query(mqd[0], mqd[1], mqd[2], mqd[3] if table is None else table,
                                         mqd[4] if lens_ is None else lens_, q_start, mq.num_kv_heads,
                                         mq.scale, mo, max_q_len=max_q_len or mq.max_q_len,
                                         max_seq_len=mq.max_seq_len)
    qs = mq.q_start.clone()
    qs_bad = qs.clone(); qs_bad[0] = 1
    expect_invalid("multi_query q_start[0] != 0", mq_call(qs_bad.to(dev)), [mo])
    qs_bad = qs.clone(); qs_bad[-1] -= 1
    expect_invalid("multi_query q_start[-1] != total_q", mq_call(qs_bad.to(dev)), [mo])
    expect_invalid("multi_query more queries than max_q_len", mq_call(qs.to(dev), max_q_len=16), [mo])
    lens_bad = mq.seq_lens.clone(); lens_bad[2] = 15     # 16 queries, 15 tokens
    expect_invalid("multi_query more queries than tokens", mq_call(qs.to(dev), lens_=lens_bad.to(dev)), [mo])
    tb_bad = mq.block_tables.clone(); tb_bad[4, 1] = mq.num_blocks + 3
    expect_invalid("multi_query table id outside the pool", mq_call(qs.to(dev), table=tb_bad.to(dev)), [mo])

    # ---- pa_decode_shared_prefix: group_start not from 0 to num_seqs, a prefix longer than a
    # member, a member whose table does not share the prefix blocks
    shd = [t.to(dev) for t in (sh.q, sh.k_cache, sh.v_cache, sh.block_tables, sh.seq_lens)]
    so = torch.full(sh.q.shape, 7.0, dtype=sh.q.dtype, device=dev)

    def sh_call(gs, pre, table=None):
        return lambda: pk.pa_decode_shared_prefix(shd[0], shd[1], shd[2], shd[3] if table is None else table,
                                                  shd[4], gs, pre, sh.num_kv_heads, sh.scale, so,
                                                  max_group_size=3, max_seq_len=sh.max_seq_len)
    gs_bad = sh.group_start.clone(); gs_bad[-1] -= 1
    expect_invalid("shared_prefix group_start[-1] != num_seqs", sh_call(gs_bad.to(dev), sh.prefix_lens.to(dev)), [so])
    pre_bad = sh.prefix_lens.clone(); pre_bad[1] = int(sh.seq_lens.max()) + 1
    expect_invalid("shared_prefix prefix longer than a member", sh_call(sh.group_start.to(dev), pre_bad.to(dev)), [so])
    tb_bad = sh.block_tables.clone()
    tb_bad[4, 0] = int(tb_bad[0, 0])                   # member 1 of group 1 leaves its prefix
    expect_invalid("shared_prefix member not sharing the prefix",
                   sh_call(sh.group_start.to(dev), sh.prefix_lens.to(dev), table=tb_bad.to(dev)), [so])

    valid = run_valid(dec, mq, sh)
    np.savez(os.path.join(out_dir, "debug_valid.npz"), **valid)
    print(json.dumps({"cases": results}), flush=True)


if __name__ == "__main__":
    main()
