"""Closed forms the pages print for KV-cache sizing and block accounting.

Test infrastructure only (see oracle/__init__.py).

Sources:
  [n1n]           explore.n1n.ai, "PagedAttention 对比传统 KV 缓存", section
                  "什么是 KV 缓存" (the Llama-2-7B sizing snippet and its 8.59 GB)
  [lpnh-2758356]  lpnh.cn/news/2758356: 1.1 (KV bytes = 2 x layers x length x
                  hidden x bytes, the 7B / 4096 / 16-request example), 2.1
                  (50 tokens in 16-token blocks), 3.1 (4 blocks instead of 256),
                  5.1 (tail waste at 150 tokens), 5.2 (pool size = reserved
                  bytes / bytes per block)
"""
from __future__ import annotations


def kv_cache_bytes(num_layers: int, num_heads: int, head_dim: int,
                   seq_len: int, batch: int, dtype_bytes: int) -> int:
    """K and V (factor 2) for every layer, head, dim, position and request."""
    return 2 * num_layers * num_heads * head_dim * seq_len * batch * dtype_bytes


def blocks_needed(n_tokens: int, block_size: int) -> int:
    """Blocks a sequence of n_tokens occupies: ceil(n / B)."""
    return -(-n_tokens // block_size)


def tail_waste_tokens(n_tokens: int, block_size: int) -> int:
    """Unused slots in the last, partly filled block."""
    return blocks_needed(n_tokens, block_size) * block_size - n_tokens


def block_bytes(block_size: int, num_layers: int, num_kv_heads: int,
                head_dim: int, dtype_bytes: int) -> int:
    """Bytes one block id pins across all layers, K and V.

    The pool-size passage lists block_size x layers x KV heads x head_dim x 2
    and drops the element width; it is restored here (a reading: the
    listed factors count elements, the size asked for is in bytes)."""
    return block_size * num_layers * num_kv_heads * head_dim * 2 * dtype_bytes


def pool_blocks(reserved_bytes: int, bytes_per_block: int) -> int:
    """Whole blocks that fit in the memory reserved for the cache."""
    return reserved_bytes // bytes_per_block
