"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI binding,
run the oracle on the same seeded inputs, compare."""

import sys
from types import SimpleNamespace

import numpy as np
import torch

import oracle
from workloads import as_numpy

# max-abs error bounds of the attention output against the float64 oracle
TOL = {"f32": 1e-5, "f16": 4e-3, "bf16": 8e-3}


def log(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def pk():
    import paged_kv_cache_351_amd as m
    m.lib()
    return m


def to_dev(b, dev="cuda"):
    d = SimpleNamespace()
    d.q = b.q.to(dev)
    d.kc = b.k_cache.to(dev)
    d.vc = b.v_cache.to(dev)
    d.bt = b.block_tables.to(dev)
    d.lens = b.seq_lens.to(dev)
    d.lens_before = b.seq_lens_before.to(dev)
    d.new_k = b.new_k.to(dev) if b.new_k is not None else None
    d.new_v = b.new_v.to(dev) if b.new_v is not None else None
    d.slots = b.slot_mapping.to(dev) if b.slot_mapping is not None else None
    d.pairs = b.cow_pairs.to(dev) if b.cow_pairs is not None else None
    return d


def gpu_decode(b, d, lens=None, max_seq_len=None, kc=None, vc=None):
    """Run pa_decode; returns the output as float64 numpy."""
    m = pk()
    lens_d = d.lens if lens is None else lens
    if max_seq_len is None:
        max_seq_len = int(lens_d.max().item()) if lens_d.numel() else 0
    out = torch.empty_like(d.q)
    m.pa_decode(d.q, d.kc if kc is None else kc, d.vc if vc is None else vc, d.bt, lens_d,
                b.num_kv_heads, b.scale, out, max_seq_len=max_seq_len)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


def oracle_decode(b, seqs=None, lens=None, kc=None, vc=None):
    lens = b.seq_lens if lens is None else lens
    return oracle.paged_decode(as_numpy(b.q), as_numpy(b.k_cache if kc is None else kc),
                               as_numpy(b.v_cache if vc is None else vc),
                               as_numpy(b.block_tables), as_numpy(lens), b.scale, b.dtype, seqs=seqs)


def allowance(ref, dtype):
    """Per-element bound: the dtype's max-abs tolerance, widened for bf16 outputs of
    magnitude >= 4 where rounding to bf16 alone can exceed it (half an ulp + 1e-5)."""
    tol = np.full(ref.shape, TOL[dtype])
    if dtype == "bf16":
        a = np.abs(ref)
        big = a >= 4
        if big.any():
            half_ulp = np.exp2(np.floor(np.log2(np.where(big, a, 1.0))) - 8)
            tol = np.where(big, half_ulp + 1e-5, tol)
    return tol


def assert_close(got, ref, dtype, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = allowance(ref, dtype)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements over tolerance, max err {err.max():.3e} "
                           f"(tol {TOL[dtype]})")
    return float(err.max()) if err.size else 0.0


def bits(t):
    """Raw bit pattern of a tensor (NaN-safe exact comparison)."""
    t = t.contiguous()
    if t.element_size() == 2:
        return t.view(torch.int16)
    return t.view(torch.int32)
