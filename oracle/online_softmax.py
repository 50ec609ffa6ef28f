"""Tiled online softmax and the log-sum-exp merge of partial states (oracle side).

These are second, independent formulations of the same attention result,
used to pin the plain definition in ``attention.py`` and to state exactly
what the GPU's split-K partitions and their merge must reproduce.

``tiled_attention`` follows "第 15 章：推理引擎与部署" §15.1 "算法详解" in its
own notation: for each row block Q_i keep m_i (running max), ℓ_i (running
sum) and O_i (unnormalised output), starting at −∞, 0, 0; for each key block
K_j, V_j::

    S_ij   = scale · Q_i K_jᵀ
    m_new  = max(m_i, rowmax(S_ij))
    α      = exp(m_i − m_new)
    P_ij   = exp(S_ij − m_new)
    ℓ_i    = α ℓ_i + rowsum(P_ij)
    O_i    = diag(α) O_i + P_ij V_j
    m_i    = m_new

and finally O_i / ℓ_i.  Keys a row may not see (beyond its causal limit or
past the context) get score −∞; a row whose state is still −∞ keeps α = 1 so
that exp(−∞ − (−∞)) never appears.

``merge_states`` combines partial states of disjoint key ranges: with
M = max_p m_p, ℓ = Σ_p ℓ_p e^{m_p − M} and O = Σ_p O_p e^{m_p − M} / ℓ.  It is
the same rescaling step as α above, applied to two finished states instead
of a state and a new block.  Partitions whose keys are all hidden (ℓ_p = 0,
m_p = −∞) contribute nothing.

Parity: pinned in tests by equality with the direct definition (to ≤1e-12 in
float64 for every tile size, ragged tails included) and by the page's own
check, tiled == standard within atol 1e-5 in float32 on N=128, d=64 with
32×32 tiles.
"""
from __future__ import annotations

import numpy as np


def partition_state(Q, K, V, scale, key_lo, key_hi, limits, block_cols):
    """Online-softmax state (m, ℓ, O unnormalised) of rows Q over keys [key_lo, key_hi).

    ``limits[r]`` is the last key position row r may see.
    """
    n, d = Q.shape
    dt = Q.dtype
    m = np.full((n, 1), -np.inf, dtype=dt)
    l = np.zeros((n, 1), dtype=dt)
    O = np.zeros((n, V.shape[1]), dtype=dt)
    lim = np.asarray(limits)
    for j in range(key_lo, key_hi, block_cols):
        je = min(j + block_cols, key_hi)
        S = (Q @ K[j:je].T) * dt.type(scale)
        vis = np.arange(j, je)[None, :] <= lim[:, None]
        S = np.where(vis, S, dt.type(-np.inf))
        m_new = np.maximum(m, S.max(axis=1, keepdims=True))
        safe = np.where(np.isneginf(m_new), dt.type(0), m_new)
        alpha = np.where(np.isneginf(m_new), dt.type(1), np.exp(m - safe))
        P = np.exp(S - safe)
        l = alpha * l + P.sum(axis=1, keepdims=True)
        O = alpha * O + P @ V[j:je]
        m = m_new
    return m, l, O


def tiled_attention(Q, K, V, scale, block_rows, block_cols, limits=None):
    """Attention of rows Q [N, d] over keys K, V [L, d] by the §15.1 tiling."""
    N = Q.shape[0]
    L = K.shape[0]
    lim = np.full(N, L - 1) if limits is None else np.asarray(limits)
    out = np.empty((N, V.shape[1]), dtype=Q.dtype)
    for i in range(0, N, block_rows):
        ie = min(i + block_rows, N)
        m, l, O = partition_state(Q[i:ie], K, V, scale, 0, L, lim[i:ie], block_cols)
        out[i:ie] = O / l
    return out


def merge_states(states):
    """Log-sum-exp merge of [(m, ℓ, O)] partial states of disjoint key ranges."""
    ms = np.stack([s[0] for s in states])          # [P, n, 1]
    M = ms.max(axis=0)
    if np.any(np.isneginf(M)):
        raise ValueError("a row sees no key in any partition")
    w = np.exp(ms - M)                              # e^{m_p - M}; 0 for empty partitions
    l = sum(wi * s[1] for wi, s in zip(w, states))
    O = sum(wi * s[2] for wi, s in zip(w, states))
    return O / l


def split_k_attention(Q, K, V, scale, part, block_cols=16, limits=None):
    """Attention of rows Q over keys split into fixed partitions of ``part`` keys, then merged."""
    N, L = Q.shape[0], K.shape[0]
    lim = np.full(N, L - 1) if limits is None else np.asarray(limits)
    states = [partition_state(Q, K, V, scale, lo, min(lo + part, L), lim, block_cols)
              for lo in range(0, L, part)]
    return merge_states(states)
