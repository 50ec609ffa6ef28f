"""Plain paged attention in float64 (oracle side).

What is computed is the textbook definition, softmax(Q Kᵀ · scale) V
("第7章：大模型部署实战" §2.2.2, the formula before the per-block pseudocode;
"第 15 章：推理引擎与部署" §15.1, the standard-attention formula).  The
per-block pseudocode on the same §2.2.2 normalises every block on its own and
adds the results; that is not the softmax over the whole context, so it is
not followed here.

Steps, per sequence ``s`` (context length ``L``, ``q_len`` query rows):

1. Gather the sequence's keys and values into contiguous float64 arrays in
   logical order: position ``p`` lives at offset ``p % 16`` of physical block
   ``block_tables[s][p // 16]`` ("第 15 章" §15.6 "PagedAttention：分页 KV
   Cache": the block table maps logical blocks to physical ones, 16 tokens per
   block by default).
2. Query row ``i`` sits at position ``L - q_len + i`` and sees keys
   ``0 .. L - q_len + i`` (decode: the new token sees itself and the whole
   cache; prefill chunk: causal inside the chunk).  ``context_lens`` counts
   the new tokens, which are in the cache before attention runs ("【自用】AI
   infra相关" part 一.2: the new K/V are put into the cache at each decode step).
3. Query head ``h`` reads KV head ``h // G`` with ``G = Hq / Hkv``: consecutive
   groups of query heads share one KV head ("大模型部署.md" §4.1 item 4 "MQA 与
   GQA").
4. ``s_j = scale · (q · k_j)``; ``w_j = exp(s_j − max s)`` (max subtraction
   leaves softmax unchanged, §15.1 "softmax(x) = softmax(x − max(x))");
   ``out = Σ w_j v_j / Σ w_j``.  The scores and the weighted sum use matrix
   products (a library primitive as one step).

Parity: pinned in tests against a single-key context (output = that value
row), identical scores (output = mean of the values), brute force with scalar
loops on tiny inputs, torch's math-backend scaled_dot_product_attention in
float64, GQA against MHA with replicated KV heads, and invariance under a
random permutation of the physical blocks.
"""
from __future__ import annotations

import numpy as np

from .layout import BLOCK, to_f64


def gather_sequence(k_pool: np.ndarray, v_pool: np.ndarray, table_row, n_keys: int, dtype: str):
    """Contiguous float64 keys and values ``[n_keys, Hkv, d]`` of one sequence, logical order."""
    nb, hkv, nchunk, blk, x = k_pool.shape
    assert blk == BLOCK
    d = nchunk * x
    n_logical = (n_keys + BLOCK - 1) // BLOCK
    K = np.empty((n_logical * BLOCK, hkv, d), dtype=np.float64)
    V = np.empty((n_logical * BLOCK, hkv, d), dtype=np.float64)
    for j in range(n_logical):
        b = int(table_row[j])
        if not 0 <= b < nb:
            raise ValueError(f"block table entry {b} outside the pool of {nb} blocks")
        # key page [Hkv, d//X, 16, X] -> [16, Hkv, d]; value page [Hkv, d, 16] -> [16, Hkv, d]
        kp = to_f64(k_pool[b], dtype).transpose(2, 0, 1, 3).reshape(BLOCK, hkv, d)
        vp = to_f64(v_pool[b], dtype).transpose(2, 0, 1)
        K[j * BLOCK:(j + 1) * BLOCK] = kp
        V[j * BLOCK:(j + 1) * BLOCK] = vp
    return K[:n_keys], V[:n_keys]


def attend_sequence(q_s: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                    rows=None) -> np.ndarray:
    """Attention of one sequence's query rows against its gathered keys/values.

    q_s: float64 ``[q_len, Hq, d]``; K, V: float64 ``[L, Hkv, d]``.
    ``rows`` optionally restricts the computation to some query rows.
    Returns float64 ``[len(rows), Hq, d]``.
    """
    q_len, hq, d = q_s.shape
    L, hkv, _ = K.shape
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = hq // hkv
    rows = np.arange(q_len) if rows is None else np.asarray(rows)
    pos = L - q_len + rows                       # position of each selected query row
    out = np.empty((len(rows), hq, d), dtype=np.float64)
    keys = np.arange(L)
    for g in range(hkv):
        Qg = q_s[rows][:, g * G:(g + 1) * G, :].reshape(len(rows) * G, d)
        S = float(scale) * (Qg @ K[:, g, :].T)   # [rows*G, L]
        visible = keys[None, :] <= np.repeat(pos, G)[:, None]
        S = np.where(visible, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        W = np.exp(S - m)
        O = (W @ V[:, g, :]) / W.sum(axis=1, keepdims=True)
        out[:, g * G:(g + 1) * G, :] = O.reshape(len(rows), G, d)
    return out


def paged_attention(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale,
                    dtype: str, tokens=None) -> np.ndarray:
    """Float64 attention output ``[T, Hq, d]`` (or only the query tokens listed in ``tokens``).

    Inputs are host copies of the exact device bytes: q as float32 or bf16
    bit patterns ``[T, Hq, d]``, the pools in the library's block layout,
    int32 block tables / context lengths / query offsets.
    """
    qf = to_f64(q, dtype)
    T, hq, d = qf.shape
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    lens = np.asarray(context_lens, dtype=np.int64)
    want = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.full((len(want), hq, d), np.nan)
    where = {int(t): i for i, t in enumerate(want)}
    for s in range(len(lens)):
        a, b = int(qsl[s]), int(qsl[s + 1])
        q_len, L = b - a, int(lens[s])
        sel = [t for t in range(a, b) if t in where]
        if not sel:
            continue
        if q_len > L:
            raise ValueError(f"sequence {s}: {q_len} query rows but only {L} keys")
        K, V = gather_sequence(k_pool, v_pool, block_tables[s], L, dtype)
        res = attend_sequence(qf[a:b], K, V, scale, rows=np.array(sel) - a)
        for t, r in zip(sel, res):
            out[where[t]] = r
    return out
