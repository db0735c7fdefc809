"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant replaces one oracle function (on the CPU, inside this test only) with
a plausible wrong version -- a dropped scale, a flipped sign, a wrong head or
block index, a per-block softmax, a swapped slot decode -- and runs the pin
tests against it.  A mutant that passes every pin would mean the pins leave that
part of the oracle unchecked.
"""

import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.cache_ops as cops
import oracle.blockmgr as bmod
import test_oracle_attention as TA
import test_oracle_cache_ops as TC
import test_oracle_swap as TS
import test_oracle_multi_query as TM


def attend_factory(kind):
    def attend(q, K, V, scale):
        Hq, D = q.shape
        L, Hkv, _ = K.shape
        g = Hq // Hkv
        out = np.zeros((Hq, D))
        if L == 0:
            return out
        for h in range(Hq):
            kv = h % Hkv if kind == "head_mod" else h // g
            sc = 1.0 if kind == "no_scale" else scale
            s = sc * (K[:, kv, :] @ q[h])
            if kind == "neg_sign":
                s = -s
            if kind == "v_from_k":
                Vh = K[:, kv, :]
            else:
                Vh = V[:, kv, :]
            p = np.exp(s - s.max())
            if kind == "no_norm":
                out[h] = p @ Vh
            elif kind == "drop_last":
                out[h] = (p[:-1] @ Vh[:-1]) / p[:-1].sum() if L > 1 else Vh[0]
            else:
                out[h] = (p @ Vh) / p.sum()
        return out
    return attend


def gather_factory(kind):
    def gather(cache, table_row, seq_len, block_size):
        t = np.arange(seq_len)
        table_row = np.asarray(table_row)
        if kind == "physical_by_index":           # ignores the table
            return cache[t // block_size, t % block_size]
        if kind == "swap_div_mod":
            return cache[table_row[t % block_size % max(1, len(table_row))], t // block_size % block_size]
        if kind == "off_by_one_block":
            return cache[table_row[np.minimum((t + 1) // block_size, len(table_row) - 1)], t % block_size]
        raise AssertionError(kind)
    return gather


def write_factory(kind):
    orig = cops.write_kv

    def write_kv(k, v, slot_mapping, k_cache, v_cache):
        if kind == "k_into_v":
            kc, vc = orig(k, v, slot_mapping, k_cache, v_cache)
            return kc, orig(k, k, slot_mapping, k_cache, v_cache)[1]
        B = k_cache.shape[1]
        kc, vc = k_cache.copy(), v_cache.copy()
        for i, s in enumerate(slot_mapping):
            if kind == "no_skip":
                s = abs(int(s))
            elif s < 0:
                continue
            b, o = (s % k_cache.shape[0], s // k_cache.shape[0]) if kind == "swap_decode" else divmod(int(s), B)
            kc[b, o % B] = k[i]
            vc[b, o % B] = v[i]
        return kc, vc
    return write_kv


def swap_factory(kind):
    orig = cops.swap_blocks

    def swap_blocks(src_k, src_v, dst_k, dst_v, pairs):
        p = [tuple(x) for x in pairs]
        if kind == "v_from_k":
            return orig(src_k, src_v, dst_k, dst_v, p)[0], orig(src_k, src_k, dst_k, dst_v, p)[1]
        if kind == "first_pair_only":
            p = p[:1]
        if kind == "reversed_pair":
            p = [(d, s) for s, d in p if d < src_k.shape[0] and s < dst_k.shape[0]]
        return orig(src_k, src_v, dst_k, dst_v, p)
    return swap_blocks


def move_factory(kind):
    orig = bmod.BlockManager._move

    def _move(self, seqs, to_cpu):
        src_ref = self.ref if to_cpu else self.cpu_ref
        before = list(src_ref)
        pairs = orig(self, seqs, to_cpu)
        dst_ref = self.cpu_ref if to_cpu else self.ref
        if kind == "count_one":                    # a shared block arrives with count 1
            for _, d in pairs:
                dst_ref[d] = 1
        elif kind == "no_release":                 # leaving sharers keep their source count
            src_free = self.free if to_cpu else self.cpu_free
            for b, _ in pairs:
                if before[b] and not src_ref[b]:
                    src_free.remove(b)
                src_ref[b] = before[b]
        elif kind == "table_not_repointed" and pairs:
            back = {d: b for b, d in pairs}
            for s in seqs:
                self.tables[s] = [back[d] for d in self.tables[s]]
        return pairs
    return _move


def multi_query_factory(kind):
    from oracle.dtypes import to_f64

    def paged_multi_query(q, k_cache, v_cache, block_tables, seq_lens, q_start, scale, dtype):
        B = k_cache.shape[1]
        out = np.zeros(q.shape)
        for s in range(len(seq_lens)):
            L = int(seq_lens[s])
            a, b = int(q_start[s]), int(q_start[s + 1])
            n = b - a
            if n > L or n < 0 or b > q.shape[0]:
                raise ValueError("bad range")
            K = to_f64(att.gather(k_cache, block_tables[s], L, B), dtype)
            V = to_f64(att.gather(v_cache, block_tables[s], L, B), dtype)
            for i in range(n):
                pos = {"from_start": i, "strict": L - n + i - 1, "no_mask": L - 1}.get(kind, L - n + i)
                if kind == "next_row":
                    pos = L - n + i
                    i_out = (i + 1) % n
                else:
                    i_out = i
                out[a + i_out] = att.attend(to_f64(q[a + i], dtype), K[:max(pos, 0) + 1],
                                            V[:max(pos, 0) + 1], scale)
        return out
    return paged_multi_query


ATTN_PINS = [
    lambda: TA.test_single_token_returns_v_exactly("f32"),
    lambda: TA.test_single_token_returns_v_exactly("bf16"),
    lambda: TA.test_zero_query_gives_mean_of_valid_rows(4),
    TA.test_one_hot_attention_selects_the_constructed_token,
    TA.test_two_tokens_match_logistic_closed_form,
    lambda: TA.test_matches_torch_sdpa_float64(8, 2),
    TA.test_unused_slots_are_never_read,
]

CACHE_PINS = [
    TC.test_worked_mapping_slots_and_next_write,
    TC.test_write_is_a_bit_copy_and_skips_negative_slots,
]


MQ_PINS = [lambda: TM.test_matches_torch_sdpa_with_offset_causal_mask(8, 2),
           TM.test_first_token_of_a_fresh_prompt_sees_only_itself,
           TM.test_causality_by_perturbing_single_rows]

SWAP_PINS = [TS.test_swap_blocks_small_example] + \
    [(lambda seed=seed: TS.test_swap_traces_read_back_every_sequence(seed)) for seed in range(3)] + \
    [TS.test_group_swap_moves_a_shared_block_once_and_keeps_outside_sharers]


def caught(pins):
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, IndexError, ValueError):
            return True
    return False


@pytest.mark.parametrize("kind", ["no_scale", "neg_sign", "head_mod", "no_norm", "v_from_k",
                                  "drop_last"])
def test_attend_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(att, "attend", attend_factory(kind))
    assert caught(ATTN_PINS), kind


@pytest.mark.parametrize("kind", ["physical_by_index", "swap_div_mod", "off_by_one_block"])
def test_gather_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(att, "gather", gather_factory(kind))
    assert caught(ATTN_PINS), kind


@pytest.mark.parametrize("kind", ["swap_decode", "no_skip", "k_into_v"])
def test_write_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(oracle, "write_kv", write_factory(kind))
    assert caught(CACHE_PINS), kind


@pytest.mark.parametrize("kind", ["v_from_k", "first_pair_only", "reversed_pair"])
def test_swap_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(oracle, "swap_blocks", swap_factory(kind))
    assert caught(SWAP_PINS), kind


@pytest.mark.parametrize("kind", ["count_one", "no_release", "table_not_repointed"])
def test_swap_bookkeeping_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(bmod.BlockManager, "_move", move_factory(kind))
    assert caught(SWAP_PINS), kind


@pytest.mark.parametrize("kind", ["from_start", "strict", "no_mask", "next_row"])
def test_multi_query_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(oracle, "paged_multi_query", multi_query_factory(kind))
    assert caught(MQ_PINS), kind


def test_unmutated_oracle_passes_every_pin():
    assert not caught(ATTN_PINS) and not caught(CACHE_PINS) and not caught(SWAP_PINS) \
        and not caught(MQ_PINS)
