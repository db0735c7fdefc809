"""Pins for the multi-query oracle (several causal queries per sequence; CPU only).

Each test ties ``oracle.paged_multi_query`` to something other than its own
formula: the decode oracle when every sequence has one query; torch's
scaled_dot_product_attention in float64 under an explicit boolean mask that
places the queries after the cached prefix; an exact special case (the first
token of a fresh prompt sees only itself); and the causal property itself,
checked by perturbing single K/V rows.  Pool slots nobody wrote hold NaN.
"""

import numpy as np
import pytest
import torch

import oracle
from test_oracle_attention import make_paged, store


def starts(ns):
    return np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)


def build(rng, lens, ns, Hq, Hkv, D, B, dtype):
    q, kc, vc, tables, lens, Klog, Vlog = make_paged(rng, lens, Hq, Hkv, D, B, dtype)
    qm = store(rng.standard_normal((int(sum(ns)), Hq, D)), dtype)
    return qm, kc, vc, tables, lens, starts(ns), Klog, Vlog


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_query_per_sequence_is_the_decode_step(dtype):
    rng = np.random.default_rng(3)
    lens = [1, 5, 16, 33, 47]
    q, kc, vc, tables, lens, qs, _, _ = build(rng, lens, [1] * 5, 8, 2, 16, 8, dtype)
    got = oracle.paged_multi_query(q, kc, vc, tables, lens, qs, 0.25, dtype)
    ref = oracle.paged_decode(q, kc, vc, tables, lens, 0.25, dtype)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 3)])
def test_matches_torch_sdpa_with_offset_causal_mask(Hq, Hkv):
    rng = np.random.default_rng(11)
    lens, ns = [9, 30, 17, 64], [3, 30, 1, 7]        # 30 = a whole prompt as one chunk
    D, B, scale = 16, 8, 0.3
    q, kc, vc, tables, lens, qs, Klog, Vlog = build(rng, lens, ns, Hq, Hkv, D, B, "f32")
    got = oracle.paged_multi_query(q, kc, vc, tables, lens, qs, scale, "f32")
    g = Hq // Hkv
    for s, (L, n) in enumerate(zip(lens, ns)):
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]].astype(np.float64)).transpose(0, 1)  # [Hq, n, D]
        K = torch.from_numpy(Klog[s]).transpose(0, 1).repeat_interleave(g, 0)      # [Hq, L, D]
        V = torch.from_numpy(Vlog[s]).transpose(0, 1).repeat_interleave(g, 0)
        pos = torch.arange(n)[:, None] + (L - n)
        mask = torch.arange(L)[None, :] <= pos                                     # [n, L]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        assert np.abs(got[qs[s]:qs[s + 1]] - ref.transpose(0, 1).numpy()).max() < 1e-12


def test_first_token_of_a_fresh_prompt_sees_only_itself():
    rng = np.random.default_rng(5)
    lens, ns = [12, 40], [12, 40]                    # the whole prompt is the query chunk
    q, kc, vc, tables, lens, qs, _, Vlog = build(rng, lens, ns, 4, 2, 16, 16, "bf16")
    out = oracle.paged_multi_query(q, kc, vc, tables, lens, qs, 0.25, "bf16")
    for s in range(2):
        # heads h and h + 1 read KV head h // 2
        assert np.array_equal(out[qs[s]], np.repeat(Vlog[s][0], 2, axis=0))


def test_causality_by_perturbing_single_rows():
    rng = np.random.default_rng(8)
    L, n, B, Hq, Hkv, D = 21, 6, 4, 4, 1, 8
    q, kc, vc, tables, lens, qs, _, _ = build(rng, [L], [n], Hq, Hkv, D, B, "f32")
    base = oracle.paged_multi_query(q, kc, vc, tables, lens, qs, 0.5, "f32")
    for t in (L - n, L - n + 2, L - 1):              # a cached position inside the chunk
        for cache in ("k", "v"):
            kc2, vc2 = kc.copy(), vc.copy()
            c = kc2 if cache == "k" else vc2
            c[tables[0, t // B], t % B] += np.float32(3.0)
            out = oracle.paged_multi_query(q, kc2, vc2, tables, lens, qs, 0.5, "f32")
            for i in range(n):
                pos = L - n + i
                if pos < t:
                    assert np.array_equal(out[i], base[i]), (t, cache, i)
                else:
                    assert not np.allclose(out[i], base[i]), (t, cache, i)


def test_rows_outside_every_sequence_stay_zero_and_bad_ranges_raise():
    rng = np.random.default_rng(2)
    q, kc, vc, tables, lens, qs, _, _ = build(rng, [5, 9], [2, 3], 4, 4, 8, 4, "f32")
    q2 = np.concatenate([q, q[:2]])                  # two trailing rows nobody owns
    out = oracle.paged_multi_query(q2, kc, vc, tables, lens, qs, 0.5, "f32")
    assert (out[5:] == 0).all()
    with pytest.raises(ValueError):
        oracle.paged_multi_query(q, kc, vc, tables, lens, np.array([0, 2, 9]), 0.5, "f32")
    with pytest.raises(ValueError):
        oracle.paged_multi_query(q, kc, vc, tables, np.array([1, 9]), qs, 0.5, "f32")
