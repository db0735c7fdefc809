"""Pins for the KV-size and block-count closed forms against every number the pages print."""

import json
import os

import pytest

import oracle

with open(os.path.join(os.path.dirname(__file__), "golden", "kv_bytes.json")) as f:
    KV_CASES = json.load(f)["cases"]
with open(os.path.join(os.path.dirname(__file__), "golden", "block_examples.json")) as f:
    BLOCKS = json.load(f)


@pytest.mark.parametrize("case", KV_CASES, ids=lambda c: c["source"][:60])
def test_kv_bytes_match_printed_values(case):
    n = oracle.kv_bytes(case["layers"], case["kv_heads"], case["head_dim"], case["dtype_bytes"],
                        case["seq_len"], case["batch"])
    assert round(n / case["unit_bytes"], case["decimals"]) == case["printed"]


def test_kv_bytes_per_token_exact_values():
    # the exact byte counts behind the printed KB figures
    assert oracle.kv_bytes_per_token(40, 40, 128, 2) == 819_200          # OPT-13B, 800 KiB
    assert oracle.kv_bytes_per_token(32, 8, 128, 2) == 131_072           # Llama-3-8B, 128 KiB
    assert oracle.kv_bytes_per_token(1, 8, 128, 2) == 4_096              # per layer, 4 KiB
    assert oracle.kv_bytes_per_token(80, 8, 128, 2) == 327_680           # Llama-2-70B, 320 KiB
    assert oracle.kv_bytes(40, 40, 128, 2, 2048) == 1_677_721_600        # OPT-13B, 2048 tokens


def test_forty_token_example():
    page = BLOCKS["forty_tokens"]["page"]
    n, B = page["num_tokens"], page["block_size"]
    assert oracle.blocks_needed(n, B) == page["num_blocks"]
    fills = [B] * (page["num_blocks"] - 1) + [oracle.last_block_fill(n, B)]
    assert fills == page["fills"]


def test_thousand_token_example():
    page = BLOCKS["thousand_tokens"]["page"]
    n, B = page["num_tokens"], page["block_size"]
    nb = oracle.blocks_needed(n, B)
    assert nb == page["num_blocks"]
    assert (nb - 1) == page["full_blocks"] and (nb - 1) * B == page["tokens_in_full_blocks"]
    assert oracle.last_block_fill(n, B) == page["last_fill"]
    assert oracle.last_block_fill(n, B) / B == page["last_fill_fraction"]


@pytest.mark.parametrize("B", [1, 8, 16, 32])
def test_block_count_brute_force(B):
    # ceil(n / B) is the least k with k*B >= n
    for n in range(0, 200):
        k = 0
        while k * B < n:
            k += 1
        assert oracle.blocks_needed(n, B) == k
        assert 0 <= k * B - n < B
        assert oracle.last_block_fill(n, B) == (n - (k - 1) * B if n else 0)
