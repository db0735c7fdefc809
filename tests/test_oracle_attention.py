"""Pins for the attention oracle (CPU only).

Each test fixes the oracle to something other than its own formula: a special
case with an exact answer, a closed form, an invariant the pages state, or a
library routine.  Together they catch a dropped scale, a sign error, a wrong
block/offset/head index, a missing cross-block normalisation or a read of an
unused pool slot (those slots hold NaN here).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import as_numpy

DT_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def store(x, dtype):
    """Round float values to the storage type; returns oracle-convention numpy."""
    return as_numpy(torch.as_tensor(np.asarray(x, dtype=np.float32)).to(DT_TORCH[dtype]))


def make_paged(rng, lens, Hq, Hkv, D, B, dtype, extra_blocks=3, q=None, K=None, V=None):
    """Scatter logical per-sequence K/V into a NaN-filled pool through random tables.

    Returns (q, kc, vc, tables, lens, Klog, Vlog) where Klog/Vlog are the exact
    float64 logical rows per sequence (what the oracle must read)."""
    nblk = [-(-L // B) for L in lens]
    NB = sum(nblk) + extra_blocks
    perm = rng.permutation(NB)
    kc = store(np.full((NB, B, Hkv, D), np.nan), dtype)
    vc = store(np.full((NB, B, Hkv, D), np.nan), dtype)
    MB = max(1, max(nblk))
    tables = np.full((len(lens), MB), -1, dtype=np.int32)
    if q is None:
        q = store(rng.standard_normal((len(lens), Hq, D)), dtype)
    Klog, Vlog = [], []
    nxt = 0
    for s, L in enumerate(lens):
        tables[s, :nblk[s]] = perm[nxt:nxt + nblk[s]]
        nxt += nblk[s]
        Ks = store(rng.standard_normal((L, Hkv, D)) if K is None else K[s], dtype)
        Vs = store(rng.standard_normal((L, Hkv, D)) if V is None else V[s], dtype)
        for t in range(L):
            kc[tables[s, t // B], t % B] = Ks[t]
            vc[tables[s, t // B], t % B] = Vs[t]
        Klog.append(oracle.to_f64(Ks, dtype))
        Vlog.append(oracle.to_f64(Vs, dtype))
    return q, kc, vc, tables, np.array(lens, dtype=np.int32), Klog, Vlog


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_token_returns_v_exactly(dtype):
    # softmax over one logit is exactly 1, so the output is that token's V row
    rng = np.random.default_rng(1)
    Hq, Hkv, D, B = 8, 2, 16, 4
    q, kc, vc, tab, lens, Klog, Vlog = make_paged(rng, [1, 1, 1], Hq, Hkv, D, B, dtype)
    out = oracle.paged_decode(q, kc, vc, tab, lens, 1 / math.sqrt(D), dtype)
    g = Hq // Hkv
    for s in range(3):
        for h in range(Hq):
            assert np.array_equal(out[s, h], Vlog[s][0, h // g])


@pytest.mark.parametrize("B", [4, 8, 16])
def test_zero_query_gives_mean_of_valid_rows(B):
    # q = 0: every logit is 0, weights are uniform 1/L over exactly the L valid tokens
    rng = np.random.default_rng(2)
    Hq, Hkv, D = 4, 4, 8
    lens = [1, B - 1, B, B + 1, 3 * B + 2]
    q0 = np.zeros((len(lens), Hq, D), dtype=np.float32)
    q, kc, vc, tab, lens, Klog, Vlog = make_paged(rng, lens, Hq, Hkv, D, B, "f32", q=q0)
    out = oracle.paged_decode(q, kc, vc, tab, lens, 0.37, "f32")
    for s in range(len(lens)):
        np.testing.assert_allclose(out[s], Vlog[s].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_one_hot_attention_selects_the_constructed_token():
    # q_h = e_h; K has a single large entry K[tau_h, h // g, h] so head h's only nonzero
    # logit is at token tau_h; everything else is 0.  Weight on tau_h is 1 - O(L e^-60).
    rng = np.random.default_rng(3)
    Hq, Hkv, D, B, L = 8, 4, 16, 4, 23
    g = Hq // Hkv
    scale = 1 / math.sqrt(D)
    tau = rng.choice(L, size=Hq, replace=False)
    q0 = np.zeros((1, Hq, D), dtype=np.float32)
    K0 = np.zeros((L, Hkv, D), dtype=np.float32)
    for h in range(Hq):
        q0[0, h, h] = 1.0
        K0[tau[h], h // g, h] = 60.0 / scale
    V0 = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    q, kc, vc, tab, lens, Klog, Vlog = make_paged(rng, [L], Hq, Hkv, D, B, "f32",
                                                  q=q0, K=[K0], V=[V0])
    out = oracle.paged_decode(q, kc, vc, tab, lens, scale, "f32")
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], V0[tau[h], h // g].astype(np.float64),
                                   rtol=0, atol=1e-20)


def test_two_tokens_match_logistic_closed_form():
    # softmax of two logits a, b gives weights sigma(a - b) and 1 - sigma(a - b)
    rng = np.random.default_rng(4)
    Hq = Hkv = 3
    D, B = 8, 16
    scale = 0.25
    q, kc, vc, tab, lens, Klog, Vlog = make_paged(rng, [2], Hq, Hkv, D, B, "f32")
    out = oracle.paged_decode(q, kc, vc, tab, lens, scale, "f32")
    qf = q[0].astype(np.float64)
    for h in range(Hq):
        a = scale * float(np.dot(Klog[0][0, h], qf[h]))
        b = scale * float(np.dot(Klog[0][1, h], qf[h]))
        w0 = 1.0 / (1.0 + math.exp(b - a))
        expect = w0 * Vlog[0][0, h] + (1.0 - w0) * Vlog[0][1, h]
        np.testing.assert_allclose(out[0, h], expect, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (8, 1), (6, 3)])
def test_matches_torch_sdpa_float64(Hq, Hkv):
    # library cross-check on unpaged tensors; GQA by repeating each KV head g times
    rng = np.random.default_rng(5)
    D, B = 32, 8
    lens = [1, 5, 8, 9, 31, 64, 70]
    q, kc, vc, tab, lens_a, Klog, Vlog = make_paged(rng, lens, Hq, Hkv, D, B, "bf16")
    scale = 1 / math.sqrt(D)
    out = oracle.paged_decode(q, kc, vc, tab, lens_a, scale, "bf16")
    g = Hq // Hkv
    qf = torch.from_numpy(oracle.to_f64(q, "bf16"))
    for s, L in enumerate(lens):
        K = torch.from_numpy(Klog[s]).repeat_interleave(g, dim=1).permute(1, 0, 2)  # [Hq, L, D]
        V = torch.from_numpy(Vlog[s]).repeat_interleave(g, dim=1).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[s][:, None, :], K.contiguous(), V.contiguous(), scale=scale)[:, 0, :]
        np.testing.assert_allclose(out[s], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_invariant_under_relabelling_physical_blocks():
    # blocks are equal-size and may sit anywhere in the pool ([PA-notes] §3)
    rng = np.random.default_rng(6)
    Hq, Hkv, D, B = 8, 2, 16, 4
    q, kc, vc, tab, lens, _, _ = make_paged(rng, [3, 9, 17], Hq, Hkv, D, B, "f16")
    out = oracle.paged_decode(q, kc, vc, tab, lens, 0.25, "f16")
    NB = kc.shape[0]
    pi = rng.permutation(NB)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    tab2 = np.where(tab >= 0, pi[np.maximum(tab, 0)], -1).astype(np.int32)
    out2 = oracle.paged_decode(q, kc2, vc2, tab2, lens, 0.25, "f16")
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("B", [4, 8, 16])
def test_blockwise_online_merge_equals_two_pass(B):
    # the pages' blockwise running-max/sum merge reaches the definition's result
    rng = np.random.default_rng(7)
    Hq, Hkv, D = 8, 4, 16
    lens = [1, B - 1, B, 2 * B + 1, 7 * B + 3]
    q, kc, vc, tab, lens_a, _, _ = make_paged(rng, lens, Hq, Hkv, D, B, "bf16")
    scale = 1 / math.sqrt(D)
    ref = oracle.paged_decode(q, kc, vc, tab, lens_a, scale, "bf16")
    for s, L in enumerate(lens):
        got = oracle.paged_decode_blockwise(q[s], kc, vc, tab[s], L, scale, "bf16")
        np.testing.assert_allclose(got, ref[s], rtol=1e-12, atol=1e-13)


def test_per_block_softmax_reading_is_rejected():
    # A softmax taken inside each block and summed over blocks (the explainer page's toy
    # code) is not attention once a sequence spans more than one block: weights then sum
    # to the number of blocks.  The oracle must differ from it there and agree for L <= B.
    rng = np.random.default_rng(8)
    Hq = Hkv = 2
    D, B = 8, 4
    q, kc, vc, tab, lens, Klog, Vlog = make_paged(rng, [4, 11], Hq, Hkv, D, B, "f32")
    out = oracle.paged_decode(q, kc, vc, tab, lens, 0.5, "f32")

    def per_block(s):
        acc = np.zeros((Hq, D))
        L = int(lens[s])
        for j in range(-(-L // B)):
            Kj, Vj = Klog[s][j * B:(j + 1) * B], Vlog[s][j * B:(j + 1) * B]
            for h in range(Hq):
                sc = 0.5 * Kj[:, h] @ q[s, h].astype(np.float64)
                w = np.exp(sc - sc.max())
                acc[h] += (w / w.sum()) @ Vj[:, h]
        return acc

    np.testing.assert_allclose(out[0], per_block(0), rtol=1e-12, atol=1e-12)
    assert np.abs(out[1] - per_block(1)).max() > 0.1


def test_empty_sequence_gives_zeros():
    rng = np.random.default_rng(9)
    q, kc, vc, tab, lens, _, _ = make_paged(rng, [0, 3], 4, 2, 8, 4, "f32")
    out = oracle.paged_decode(q, kc, vc, tab, lens, 0.5, "f32")
    assert np.array_equal(out[0], np.zeros((4, 8)))
    assert np.isfinite(out[1]).all()
    assert np.array_equal(oracle.paged_decode_blockwise(q[0], kc, vc, tab[0], 0, 0.5, "f32"),
                          np.zeros((4, 8)))


def test_unused_slots_are_never_read():
    # every unused slot and every padding table entry holds NaN / -1; results stay finite
    rng = np.random.default_rng(10)
    q, kc, vc, tab, lens, _, _ = make_paged(rng, [5, 16, 33], 4, 4, 8, 16, "bf16",
                                            extra_blocks=10)
    out = oracle.paged_decode(q, kc, vc, tab, lens, 0.3, "bf16")
    assert np.isfinite(out).all()


def test_bf16_widening_is_exact():
    vals = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0, -0.0], dtype=np.float32)
    bits = store(vals, "bf16")
    back = oracle.to_f64(bits, "bf16")
    ref = torch.tensor(vals).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, ref)
    assert oracle.to_f64(np.array([0x3F80, 0xC020], dtype=np.uint16), "bf16").tolist() == [1.0, -2.5]
