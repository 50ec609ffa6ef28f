"""Cache write through a slot mapping, and copy-on-write block copies (oracle side).

``reshape_and_cache``: every new token ``t`` carries a slot number; its key
and value rows go to offset ``slot % 16`` of physical block ``slot // 16`` for
every KV head.  Slots index the KV storage directly, as SGLang's
``out_cache_loc`` does ("大模型部署.md" §2.4 item 4, the generation-stage
flow), and a decode step stores the new K/V into the cache ("【自用】AI
infra相关" part 一.2).  A negative slot marks a padding token and is skipped.
Slots must be distinct and inside the pool; the oracle raises otherwise.

``copy_blocks``: for each (src, dst) pair, the whole key and value page of
``src`` (all KV heads) is copied onto ``dst`` — the private copy that
copy-on-write makes before a sequence writes into a shared block
("大模型部署.md" §2.1 item 3, ``append_slots`` returning the
``(old, new)`` block pair; item 4 "写时复制").  Destinations must be distinct
and disjoint from sources, which is what copy-on-write produces (the copy
always lands in a freshly allocated block).

Both operate on numpy copies of the pool bytes and are compared with the GPU
bit for bit.  Parity: pinned by round trips through ``layout`` readers, by
the untouched-bytes invariant and by a hand-indexed golden fixture.
"""
from __future__ import annotations

import numpy as np

from .layout import BLOCK, set_key_row, set_value_row


def reshape_and_cache(key, value, k_pool, v_pool, slot_mapping, inplace=False):
    """Pools with token rows of ``key``/``value`` [T, Hkv, d] stored at their slots.

    Returns new pools, or writes into the given ones when ``inplace``.
    """
    if not inplace:
        k_pool = np.array(k_pool, copy=True)
        v_pool = np.array(v_pool, copy=True)
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots[slots >= 0]
    if live.size and (live.max() >= nb * BLOCK):
        raise ValueError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slots")
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), BLOCK)
        for h in range(hkv):
            set_key_row(k_pool, block, h, offset, key[t, h])
            set_value_row(v_pool, block, h, offset, value[t, h])
    return k_pool, v_pool


def copy_blocks(k_pool, v_pool, pairs, inplace=False):
    """Pools where every destination block holds a copy of its source block (new, or in place)."""
    if not inplace:
        k_pool = np.array(k_pool, copy=True)
        v_pool = np.array(v_pool, copy=True)
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    nb = k_pool.shape[0]
    if pairs.size:
        if pairs.min() < 0 or pairs.max() >= nb:
            raise ValueError("block id outside the pool")
        dst = pairs[:, 1]
        if np.unique(dst).size != dst.size or np.intersect1d(dst, pairs[:, 0]).size:
            raise ValueError("destinations must be distinct and disjoint from sources")
    for src, dst in pairs:
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]
    return k_pool, v_pool
