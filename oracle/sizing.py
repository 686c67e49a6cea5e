"""KV-cache size arithmetic (test infrastructure only; see package docstring).

Source: "KV Cache 原理与 PagedAttention", §一, the 显存占用公式 paragraph: one
layer's cache holds a K and a V vector per KV head per token, so its size is
2 x num_kv_heads x seq_len x head_dim x dtype_bytes, and the whole model's is
that times the layer count.  The bjdmk.com.cn article (§2.2) states the same
count per token over all layers.

All results are exact Python integers.
"""

from __future__ import annotations

import math


def kv_bytes_per_layer(num_kv_heads: int, seq_len: int, head_dim: int,
                       dtype_bytes: int) -> int:
    """Bytes of K plus V for one layer and one sequence of ``seq_len`` tokens."""
    return 2 * num_kv_heads * seq_len * head_dim * dtype_bytes


def kv_bytes_total(num_layers: int, num_kv_heads: int, seq_len: int,
                   head_dim: int, dtype_bytes: int) -> int:
    """Bytes of K plus V over all layers for one sequence."""
    return num_layers * kv_bytes_per_layer(num_kv_heads, seq_len, head_dim,
                                           dtype_bytes)


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       dtype_bytes: int) -> int:
    """Bytes one token adds to the cache over all layers."""
    return kv_bytes_total(num_layers, num_kv_heads, 1, head_dim, dtype_bytes)


def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` tokens occupies: the last block may
    be partly empty, never more than one block is partly empty
    ("KV Cache 原理与 PagedAttention", §三 收益 table, internal-fragmentation row).
    """
    return math.ceil(num_tokens / block_size) if num_tokens > 0 else 0


def paged_pool_bytes(num_layers: int, num_blocks: int, block_size: int,
                     num_kv_heads: int, head_dim: int, elem_bytes: int,
                     per_token_head_scales: bool = False) -> int:
    """Payload bytes of a paged pool: K and V for every slot of every block
    of every layer, plus (INT8 per-token-head storage) one fp32 scale per
    (layer, block, kv head, slot) for K and another for V.  Region alignment
    padding is not counted here; ``layout.region_offsets`` adds it.
    """
    kv = 2 * num_layers * num_blocks * block_size * num_kv_heads * head_dim * elem_bytes
    if per_token_head_scales:
        kv += 2 * num_layers * num_blocks * block_size * num_kv_heads * 4
    return kv
