"""Plain CPU oracle for paged decode attention and its cache operations.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: it exists so that tests, the smoke check and the
benchmark's CPU-baseline leg can compute what the GPU path must reproduce.  It
shares no code, table or constant with the HIP library in
``paged_kv_cache_351_amd`` and never imports it.

Everything here is written from three web pages about PagedAttention.  They are
cited by short key plus section:

  [PA-notes]     "LLM 注意力与计算内核精读笔记 · 05 PagedAttention 与 KV 显存管理"
                 (study notes on Kwon et al., SOSP 2023) -- the authority on what
                 is computed.
  [vLLM-what]    "vLLM 是什么 PagedAttention 解决了什么"
  [PA-explainer] "PagedAttention：分页注意力——推理引擎的显存革命"

Arithmetic is numpy float64.  Stored half-precision values are widened exactly
(bfloat16 arrives as its raw uint16 bit pattern, float16 as numpy float16).

Parity status of each function is stated in its module; every function here is
pinned by ``tests/test_oracle_*.py`` against page values, closed forms,
invariants or a library routine.
"""

from .dtypes import DTYPES, to_f64, from_f32_bits
from .attention import gather, attend, paged_decode, paged_decode_blockwise, paged_multi_query
from .cache_ops import write_kv, copy_blocks, swap_blocks
from .blockmgr import BlockManager, OutOfBlocks
from .kv_bytes import kv_bytes_per_token, kv_bytes, blocks_needed, last_block_fill

__all__ = [
    "DTYPES", "to_f64", "from_f32_bits",
    "gather", "attend", "paged_decode", "paged_decode_blockwise", "paged_multi_query",
    "write_kv", "copy_blocks", "swap_blocks",
    "BlockManager", "OutOfBlocks",
    "kv_bytes_per_token", "kv_bytes", "blocks_needed", "last_block_fill",
]
