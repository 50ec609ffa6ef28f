"""Block-count and KV-size arithmetic (oracle side).

* ``blocks_for(L, P)`` — a request of L tokens needs ⌈L / P⌉ blocks of P
  tokens ("第7章：大模型部署实战" §2.2.1 "块分配机制").
* ``last_block_waste(L, P)`` — only the last block holds unused slots:
  P·⌈L/P⌉ − L ("大模型部署.md" §2.1 item 4: only the last block wastes memory;
  "【自用】AI infra相关" part 二, internal fragmentation example).
* ``kv_cache_bytes(L, h, d, b)`` — 2 × L × h × d_head × b × 2 bytes: K and V,
  L tokens, h heads of d_head, batch b, 2-byte elements ("第7章" §2.1).
* ``kv_bytes_per_token(layers, n_kv, d, p)`` — 2 × layers × N_kv × D_head ×
  P_byte ("第 15 章：推理引擎与部署" §15.6 "KV Cache 大小计算").

Parity: pinned by the worked numbers the pages print (tests/golden).
"""
from __future__ import annotations


def blocks_for(n_tokens: int, block_size: int) -> int:
    if n_tokens < 0 or block_size <= 0:
        raise ValueError("negative length or non-positive block size")
    return (n_tokens + block_size - 1) // block_size


def last_block_waste(n_tokens: int, block_size: int) -> int:
    return block_size * blocks_for(n_tokens, block_size) - n_tokens


def kv_cache_bytes(seq_len: int, heads: int, head_dim: int, batch: int, elem_bytes: int = 2) -> int:
    return 2 * seq_len * heads * head_dim * batch * elem_bytes


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * kv_heads * head_dim * elem_bytes


def tokens_held(num_blocks: int, block_size: int) -> int:
    return num_blocks * block_size
