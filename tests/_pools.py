"""Host-side (numpy) pools for CPU tests: logical K/V placed into the block layout.

Test input construction only: draws values, rounds them to bfloat16 bit
patterns when asked, and stores every sequence's logical rows into its
physical blocks through the oracle's layout writers (which the golden
offset fixture pins).  Unreferenced blocks hold unrelated random values.
"""
import numpy as np

from oracle import layout

BLOCK = 16


def bf16_bits(x):
    """Round float32 values to bfloat16 (nearest even) and return the uint16 bit patterns."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def raw(x, dtype):
    return np.asarray(x, dtype=np.float32) if dtype == "f32" else bf16_bits(x)


def empty_pools(rng, dtype, nb, hkv, d):
    x = layout.elems_per_16_bytes(dtype)
    kp = raw(rng.standard_normal((nb, hkv, d // x, BLOCK, x)).astype(np.float32), dtype)
    vp = raw(rng.standard_normal((nb, hkv, d, BLOCK)).astype(np.float32), dtype)
    return kp, vp


def place(kp, vp, table_row, K_raw, V_raw):
    """Store logical rows K_raw/V_raw [L, Hkv, d] of one sequence into its blocks."""
    L, hkv, _ = K_raw.shape
    for p in range(L):
        b, o = int(table_row[p // BLOCK]), p % BLOCK
        for h in range(hkv):
            layout.set_key_row(kp, b, h, o, K_raw[p, h])
            layout.set_value_row(vp, b, h, o, V_raw[p, h])


def build_case(seed, dtype, hq, hkv, d, lens, qlens, slack=4, scale_q=1.0):
    """Random ragged batch with known logical K/V. Returns a dict of host arrays."""
    rng = np.random.default_rng(seed)
    lens = [int(L) for L in lens]
    nblk = [(L + BLOCK - 1) // BLOCK for L in lens]
    nb = sum(nblk) + slack
    perm = rng.permutation(nb).astype(np.int32)
    mb = max(max(nblk), 1)
    tables = np.full((len(lens), mb), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[off:off + n]
        off += n
    kp, vp = empty_pools(rng, dtype, nb, hkv, d)
    Klog, Vlog = [], []
    for s, L in enumerate(lens):
        K_raw = raw(rng.standard_normal((L, hkv, d)).astype(np.float32), dtype)
        V_raw = raw(rng.standard_normal((L, hkv, d)).astype(np.float32), dtype)
        place(kp, vp, tables[s], K_raw, V_raw)
        Klog.append(layout.to_f64(K_raw, dtype))
        Vlog.append(layout.to_f64(V_raw, dtype))
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    q = raw((scale_q * rng.standard_normal((T, hq, d))).astype(np.float32), dtype)
    return dict(dtype=dtype, kp=kp, vp=vp, tables=tables, lens=np.array(lens, np.int32),
                qsl=qsl, q=q, Klog=Klog, Vlog=Vlog, hq=hq, hkv=hkv, d=d,
                scale=float(np.float32(1.0 / np.sqrt(d))))
