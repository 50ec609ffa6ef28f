"""Pins of the oracle's cache write, block copy, allocator mirror and size helpers."""
import json
import math
import os

import numpy as np
import pytest

from oracle import allocator as A
from oracle import cache_ops, layout, sizes
from tests._pools import empty_pools, raw
from tests.conftest import GOLDEN


def load(name):
    return json.load(open(os.path.join(GOLDEN, name)))


# ---------------------------------------------------------------- layout / cache write

@pytest.mark.parametrize("case", load("layout_offsets.json")["cases"])
def test_layout_flat_offsets(case):
    dt = case["dtype"]
    x = layout.elems_per_16_bytes(dt)
    nb, hkv, d = case["num_blocks"], case["kv_heads"], case["head_dim"]
    np_dt = np.float32 if dt == "f32" else np.uint16
    kp = np.zeros((nb, hkv, d // x, 16, x), np_dt)
    vp = np.zeros((nb, hkv, d, 16), np_dt)
    row = np.arange(1, d + 1).astype(np_dt)
    layout.set_key_row(kp, case["block"], case["head"], case["offset"], row)
    layout.set_value_row(vp, case["block"], case["head"], case["offset"], row)
    assert list(np.flatnonzero(kp.reshape(-1))) == case["key_offsets"]
    assert list(np.flatnonzero(vp.reshape(-1))) == case["value_offsets"]
    assert list(kp.reshape(-1)[case["key_offsets"]]) == list(row)
    assert list(vp.reshape(-1)[case["value_offsets"]]) == list(row)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cache_write_round_trip_and_untouched_bytes(dtype):
    rng = np.random.default_rng(1)
    nb, hkv, d, T = 6, 3, 32, 40
    kp, vp = empty_pools(rng, dtype, nb, hkv, d)
    key = raw(rng.standard_normal((T, hkv, d)).astype(np.float32), dtype)
    val = raw(rng.standard_normal((T, hkv, d)).astype(np.float32), dtype)
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[[3, 17]] = -1                                      # padding tokens
    k2, v2 = cache_ops.reshape_and_cache(key, val, kp, vp, slots)
    touched_k = np.zeros(kp.shape, bool)
    touched_v = np.zeros(vp.shape, bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), 16)
        for h in range(hkv):
            assert np.array_equal(layout.key_row(k2, b, h, o), key[t, h])
            assert np.array_equal(layout.value_row(v2, b, h, o), val[t, h])
            touched_k[b, h, :, o, :] = True
            touched_v[b, h, :, o] = True
    assert np.array_equal(k2[~touched_k], kp[~touched_k])
    assert np.array_equal(v2[~touched_v], vp[~touched_v])
    assert touched_k.sum() == (T - 2) * hkv * d


def test_cache_write_rejects_bad_slots():
    rng = np.random.default_rng(2)
    kp, vp = empty_pools(rng, "f32", 2, 1, 8)
    key = np.zeros((2, 1, 8), np.float32)
    with pytest.raises(ValueError):
        cache_ops.reshape_and_cache(key, key, kp, vp, np.array([3, 3]))
    with pytest.raises(ValueError):
        cache_ops.reshape_and_cache(key, key, kp, vp, np.array([0, 32]))


def test_copy_blocks_copies_whole_pages_only():
    rng = np.random.default_rng(3)
    kp, vp = empty_pools(rng, "bf16", 8, 2, 64)
    k2, v2 = cache_ops.copy_blocks(kp, vp, [(1, 5), (1, 6), (3, 0)])
    for s, d in [(1, 5), (1, 6), (3, 0)]:
        assert np.array_equal(k2[d], kp[s]) and np.array_equal(v2[d], vp[s])
    for b in (1, 2, 3, 4, 7):
        assert np.array_equal(k2[b], kp[b]) and np.array_equal(v2[b], vp[b])
    with pytest.raises(ValueError):
        cache_ops.copy_blocks(kp, vp, [(1, 5), (5, 2)])       # dst reused as src


# ---------------------------------------------------------------- sizes

def test_printed_size_examples():
    fx = load("kv_size_examples.json")
    for e in fx["kv_cache_bytes"]:
        assert sizes.kv_cache_bytes(e["seq_len"], e["heads"], e["head_dim"], e["batch"],
                                    e["elem_bytes"]) == e["bytes"]
    for e in fx["kv_bytes_per_token"]:
        assert sizes.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"],
                                        e["elem_bytes"]) == e["bytes"]
    for e in fx["tokens_held"]:
        assert sizes.tokens_held(e["num_blocks"], e["block_size"]) == e["tokens"]
    for e in fx["last_block_waste"]:
        assert sizes.last_block_waste(e["tokens"], e["block_size"]) == e["wasted_slots"]


def test_block_count_is_ceiling():
    for L in range(0, 40001):
        assert sizes.blocks_for(L, 16) == math.ceil(L / 16)
        assert 0 <= sizes.last_block_waste(L, 16) <= 15


# ---------------------------------------------------------------- allocator mirror

def test_page_block_size_4_example():
    fx = load("block_size4_example.json")
    a = A.Allocator(fx["num_blocks"], fx["block_size"], 0.0, fx["initial_free_order"])
    a.create("req", fx["prompt_tokens"])
    assert a.block_table("req") == fx["table_after_prompt"]
    slot, cow = a.append_slot("req")
    assert a.block_table("req") == fx["table_after_fifth_token"]
    assert slot == fx["slot_of_fifth_token"] and cow is None


def test_copy_on_write_only_for_shared_partial_block():
    a = A.Allocator(16, 4)
    a.create(0, 6)                       # blocks: 15, 14 (second block half full)
    for c in (1, 2, 3):
        a.fork(0, c)
    assert a.ref[15] == 4 and a.ref[14] == 4
    pairs = []
    for s in (0, 1, 2, 3):
        slot, cow = a.append_slot(s)
        pairs.append(cow)
        assert slot // 4 == a.block_table(s)[1] and slot % 4 == 2
    # three branches copy the shared last block; the fourth finds itself its only owner
    assert pairs[:3] == [(14, 13), (14, 12), (14, 11)] and pairs[3] is None
    assert a.ref[14] == 1 and a.ref[15] == 4
    assert [a.block_table(s)[1] for s in range(4)] == [13, 12, 11, 14]


def test_aligned_prompt_forks_without_copy():
    a = A.Allocator(16, 4)
    a.create(0, 8)
    a.fork(0, 1)
    s0, c0 = a.append_slot(0)
    s1, c1 = a.append_slot(1)
    assert c0 is None and c1 is None and s0 // 4 != s1 // 4


def test_can_allocate_statuses_and_watermark():
    a = A.Allocator(100, 16, watermark=0.1)          # 10 watermark blocks
    assert a.can_allocate(16 * 91) == A.NEVER
    assert a.can_allocate(16 * 90) == A.OK
    a.create(0, 16 * 50)
    assert a.can_allocate(16 * 41) == A.LATER
    assert a.can_allocate(16 * 40) == A.OK


def test_exhaustion_leaves_state_unchanged():
    a = A.Allocator(4, 16)
    a.create(0, 40)                                   # 3 blocks
    before = (list(a.free), list(a.ref))
    with pytest.raises(A.NoBlocks):
        a.create(1, 33)
    assert (list(a.free), list(a.ref)) == before and 1 not in a.tables


def test_free_pushes_in_logical_order():
    a = A.Allocator(8, 16)
    a.create(0, 48)                                   # pops 7, 6, 5
    a.free_seq(0)
    assert a.free[-3:] == [7, 6, 5]


def test_random_operation_invariants():
    rng = np.random.default_rng(7)
    a = A.Allocator(64, 4, initial_free_order=rng.permutation(64))
    nxt = 0
    for _ in range(3000):
        op = rng.integers(0, 4)
        live = list(a.tables)
        try:
            if op == 0 or not live:
                a.create(nxt, int(rng.integers(0, 20)))
                nxt += 1
            elif op == 1:
                a.fork(live[rng.integers(len(live))], nxt)
                nxt += 1
            elif op == 2:
                a.append_slot(live[rng.integers(len(live))])
            else:
                a.free_seq(live[rng.integers(len(live))])
        except A.NoBlocks:
            pass
        held = [b for t in a.tables.values() for b in t]
        assert sum(a.ref) == len(held)
        assert len(a.free) + sum(1 for r in a.ref if r > 0) == 64
        assert not set(a.free) & set(held)
        for s, t in a.tables.items():
            assert len(t) == (a.ntok[s] + 3) // 4


def test_bf16_widening_matches_torch_and_known_encodings():
    import torch
    # bfloat16 is the top 16 bits of an IEEE float32: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3F00 = 0.5
    known = np.array([0x3F80, 0xC000, 0x3F00, 0x0000, 0x4049], np.uint16)
    got = layout.to_f64(known, "bf16")
    assert list(got[:4]) == [1.0, -2.0, 0.5, 0.0] and abs(got[4] - 3.140625) == 0
    bits = np.random.default_rng(0).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                     # skip inf / nan encodings
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(layout.to_f64(bits, "bf16"), ref)


def test_inplace_cache_ops_match_functional_ones():
    rng = np.random.default_rng(4)
    kp, vp = empty_pools(rng, "bf16", 5, 2, 64)
    key = raw(rng.standard_normal((7, 2, 64)).astype(np.float32), "bf16")
    slots = np.array([3, 17, 40, -1, 79, 0, 33])
    k1, v1 = cache_ops.reshape_and_cache(key, key, kp, vp, slots)
    k2, v2 = kp.copy(), vp.copy()
    cache_ops.reshape_and_cache(key, key, k2, v2, slots, inplace=True)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    k3, v3 = cache_ops.copy_blocks(k1, v1, [(1, 4)])
    cache_ops.copy_blocks(k2, v2, [(1, 4)], inplace=True)
    assert np.array_equal(k3, k2) and np.array_equal(v3, v2)
