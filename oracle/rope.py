"""Rotary position embedding applied before the cache write (oracle side; test infrastructure).

The pages apply the rotation as ``apply_rope(x, cos, sin)`` to q and k before
attention, and describe the fused form that rotates them in registers on the
way through the kernel ("第 15 章：推理引擎与部署" §15.3, RoPE fused with
attention; "DeepSpeed-FastGen 深度解析" §6, a QKV kernel fused with the rotary
embedding and the blocked KV layout).  They print no formula; the plain
reading used here is the rotate-half form: for a row x of head_dim d and a
position p with table rows c = cos[p], s = sin[p] (d/2 entries each),

    x'[i]       = x[i] c[i] − x[i + d/2] s[i]
    x'[i + d/2] = x[i + d/2] c[i] + x[i] s[i]        (0 <= i < d/2)

i.e. each pair (x[i], x[i + d/2]) read as the complex number x[i] + j x[i+d/2]
is multiplied by c[i] + j s[i].  The tables are inputs (the caller's
cos(p θ_i), sin(p θ_i)); this module only applies them, in float64.

Parity: pinned by the identity at angle 0, a quarter turn, the complex
product form, norm preservation, the dependence of q'·k' on the position
difference only, and additivity of angles.
"""
from __future__ import annotations

import numpy as np


def rope(x: np.ndarray, positions: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x: [T, H, d] (float), positions: [T] int, cos/sin: [max_pos, d/2].  Returns float64 [T, H, d]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    c = np.asarray(cos, dtype=np.float64)[np.asarray(positions)][:, None, :]   # [T, 1, d/2]
    s = np.asarray(sin, dtype=np.float64)[np.asarray(positions)][:, None, :]
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), rounded once, to nearest, ties to even:
    x = m 2^e with 0.5 <= |m| < 1, and bfloat16 keeps 8 significant bits, so the
    result is rint(m 2^8) 2^(e-8) (exact in float32, whose top half is the pattern)."""
    f = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(f)
    v = np.ldexp(np.rint(m * 256.0), e - 8)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
