"""Reading and writing single token rows of the paged K/V pools (oracle side).

The pools are the byte images the library works on, viewed as numpy arrays:

* key pool   ``[num_blocks, kv_heads, head_dim // X, 16, X]``
* value pool ``[num_blocks, kv_heads, head_dim, 16]``

with ``X = 16 // itemsize`` (8 for bfloat16, 4 for float32).  Token ``o`` of
physical block ``b`` and KV head ``h`` therefore keeps its key as the
``head_dim // X`` runs ``key[b, h, c, o, :]`` and its value as the column
``value[b, h, :, o]``.  This is a storage format: a (block, head) page is the
fixed-size unit the pages describe ("第 15 章：推理引擎与部署", §15.6
"PagedAttention：分页 KV Cache": 16 tokens per block, reached through the block
table), only the order of elements inside the page is the library's choice.

bfloat16 pools are held as ``uint16`` bit patterns; ``to_f64`` widens them
exactly (a bfloat16 is the top half of a float32).

Parity: pinned in tests by round trips (write then read back in logical
order) and by a hand-indexed golden fixture of flat element offsets.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def elems_per_16_bytes(dtype: str) -> int:
    return 16 // (4 if dtype == "f32" else 2)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of float32 arrays or bfloat16 bit patterns (uint16) to float64."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def key_row(k_pool: np.ndarray, block: int, head: int, offset: int) -> np.ndarray:
    """The head_dim key elements of one token (raw storage type)."""
    return k_pool[block, head, :, offset, :].reshape(-1)


def value_row(v_pool: np.ndarray, block: int, head: int, offset: int) -> np.ndarray:
    """The head_dim value elements of one token (raw storage type)."""
    return v_pool[block, head, :, offset]


def set_key_row(k_pool: np.ndarray, block: int, head: int, offset: int, row: np.ndarray) -> None:
    nchunk, x = k_pool.shape[2], k_pool.shape[4]
    k_pool[block, head, :, offset, :] = np.asarray(row).reshape(nchunk, x)


def set_value_row(v_pool: np.ndarray, block: int, head: int, offset: int, row: np.ndarray) -> None:
    v_pool[block, head, :, offset] = row
