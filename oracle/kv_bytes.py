"""Closed forms for KV-cache size and block bookkeeping (oracle, test infrastructure).

* Bytes of K and V for one token:  2 × layers × kv_heads × head_dim × bytes
  ([vLLM-what] "1）KV cache 显存估算" gives the formula with seq_len and batch
  factors; [PA-notes] §2 and §9.1 use it for OPT-13B with hidden = heads ×
  head_dim).
* Blocks for n tokens: ceil(n / B) ([PA-explainer] "动态分配";
  [PA-notes] §9.2 and §12 题1).
* Fill of the last block: n - (ceil(n / B) - 1) × B.

Pinned against every worked number the pages print
(tests/golden/kv_bytes.json, tests/golden/block_examples.json).
"""


def kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes):
    return 2 * layers * kv_heads * head_dim * dtype_bytes


def kv_bytes(layers, kv_heads, head_dim, dtype_bytes, seq_len, batch=1):
    return kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes) * seq_len * batch


def blocks_needed(num_tokens, block_size):
    return (num_tokens + block_size - 1) // block_size


def last_block_fill(num_tokens, block_size):
    if num_tokens == 0:
        return 0
    return num_tokens - (blocks_needed(num_tokens, block_size) - 1) * block_size
