"""Checks of a rotary cache write against the oracle (shared by the emulator and GPU tests).

The rotation is floating-point work, so the library's float32 evaluation is
compared with the exact (float64) rotation rounded once to the storage type:
each element may differ by the rounding of the float32 evaluation, bounded by
2^-22 (|x| + |y|) for the pair (x, y) it mixes, plus one unit in the last place
of the stored type (a float32 result on the other side of a rounding
boundary).  Values and untouched pool bytes must be bit-exact.
"""
import numpy as np

from oracle import cache_ops, layout
from oracle.rope import bf16_round, rope


def ulp(v, dtype):
    mant = 7 if dtype == "bf16" else 23
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - mant), 2.0 ** -133)


def expected(dtype, q, key, val, kp, vp, slots, positions, cos, sin):
    """(q', k_pool', v_pool', bound on |q' - got|, bound per rotated key row) from the oracle."""
    qf, kf = layout.to_f64(q, dtype), layout.to_f64(key, dtype)
    qr, kr = rope(qf, positions, cos, sin), rope(kf, positions, cos, sin)
    store = (lambda x: bf16_round(x)) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    def bound(x, r):
        h = x.shape[-1] // 2
        pair = np.abs(x[..., :h]) + np.abs(x[..., h:])
        return np.concatenate([pair, pair], axis=-1) * 2.0 ** -22 + ulp(r, dtype)
    kp2, vp2 = cache_ops.reshape_and_cache(store(kr), val, kp, vp, slots)
    return store(qr), kp2, vp2, bound(qf, qr), bound(kf, kr)


def check(dtype, got_q, got_k, got_v, q, key, val, kp, vp, slots, positions, cos, sin):
    q_ref, k_ref, v_ref, qb, kb = expected(dtype, q, key, val, kp, vp, slots, positions, cos, sin)
    assert np.array_equal(got_v, v_ref), "value pool differs"
    dq = np.abs(layout.to_f64(got_q, dtype) - layout.to_f64(q_ref, dtype))
    assert (dq <= qb).all(), f"rotated q off by {float((dq / qb).max()):.2f} of its bound"
    same = np.mean(got_q == q_ref)
    # key rows that were written: compare with tolerance, then the rest of the pool bit for bit
    gk, rk = got_k.copy(), k_ref.copy()
    for t, sl in enumerate(np.asarray(slots)):
        if sl < 0 or sl >= kp.shape[0] * 16:
            continue
        b, o = int(sl) // 16, int(sl) % 16
        for h in range(key.shape[1]):
            g = layout.to_f64(layout.key_row(gk, b, h, o), dtype)
            r = layout.to_f64(layout.key_row(rk, b, h, o), dtype)
            assert (np.abs(g - r) <= kb[t, h]).all(), f"rotated key of token {t} head {h}"
            layout.set_key_row(gk, b, h, o, layout.key_row(rk, b, h, o))
    assert np.array_equal(gk, rk), "key pool differs outside the written rows"
    return same
