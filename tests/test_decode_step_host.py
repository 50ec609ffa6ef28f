"""Host half of the decode step (pa_decode_step_stage) against the oracle's
allocator mirror, and the argument checks of pa_decode_step (no GPU needed:
every case below returns before anything is enqueued)."""
import ctypes

import numpy as np
import pytest

from oracle import allocator as mirror_alloc


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_57_amd as pa
    return pa


def layout(n, cols):
    """Byte offsets of the staging layout written out from its description in pa.h."""
    lens = 8 * n
    qsl = 12 * n
    pairs = (16 * n + 4 + 7) // 8 * 8
    tables = pairs + 8 * n
    return lens, qsl, pairs, tables, tables + 4 * n * cols


def test_staging_bytes_formula(pa):
    for n, m in [(1, 1), (3, 7), (64, 300), (1024, 256)]:
        assert pa.pa_decode_step_staging_bytes(n, m) == layout(n, m)[4]
    assert pa.pa_decode_step_staging_bytes(0, 5) == 0
    assert pa.pa_decode_step_staging_bytes(4, 0) == 0


def test_stage_matches_mirror_over_steps(pa):
    """4 prompts x 3 branches (forks: copy-on-write of the shared partial page), 40 steps;
    every step the staged slots, lengths, query starts, copy pairs and tables equal the
    mirror's, byte for byte."""
    rng = np.random.default_rng(11)
    NB, P, B, M = 256, 4, 3, 40
    order = rng.permutation(NB).astype(np.int32)
    alloc = pa.Allocator(NB, 16, 0.0, order)
    mirror = mirror_alloc.Allocator(NB, 16, 0.0, order)
    plens = rng.integers(5, 200, size=P)
    for p, L in enumerate(plens):
        alloc.create(p * B, int(L))
        mirror.create(p * B, int(L))
        for b in range(1, B):
            alloc.fork(p * B, p * B + b)
            mirror.fork(p * B, p * B + b)
    ids = [p * B + b for p in range(P) for b in range(B)]
    n = len(ids)
    buf = np.zeros(pa.pa_decode_step_staging_bytes(n, M), np.uint8)
    total_cow = 0
    for step in range(40):
        buf[:] = 0xAB
        ncow, mx, cols, used = pa.pa_decode_step_stage(alloc, ids, M, buf)
        want_slots, want_pairs = [], []
        for s in ids:
            sl, cow = mirror.append_slot(s)
            want_slots.append(sl)
            if cow:
                want_pairs.append(cow)
        lens = np.array([mirror.ntok[s] for s in ids], np.int32)
        o_lens, o_qsl, o_pairs, o_tab, end = layout(n, cols)
        assert (mx, cols, used) == (int(lens.max()), (int(lens.max()) + 15) // 16, end), step
        assert ncow == len(want_pairs), step
        total_cow += ncow
        assert np.array_equal(buf[:o_lens].view(np.int64), np.array(want_slots, np.int64)), step
        assert np.array_equal(buf[o_lens:o_qsl].view(np.int32), lens), step
        assert np.array_equal(buf[o_qsl:o_qsl + 4 * (n + 1)].view(np.int32), np.arange(n + 1, dtype=np.int32))
        got_pairs = buf[o_pairs:o_pairs + 8 * ncow].view(np.int32).reshape(-1, 2)
        assert [tuple(x) for x in got_pairs] == want_pairs, step
        want_tab = np.full((n, cols), -1, np.int32)
        for i, s in enumerate(ids):
            t = mirror.block_table(s)
            want_tab[i, :len(t)] = t
        assert np.array_equal(buf[o_tab:end].view(np.int32).reshape(n, cols), want_tab), step
        assert alloc.num_free() == mirror.num_free()
    assert total_cow > 0


def test_stage_errors_leave_the_allocator_unchanged(pa):
    NB = 64
    alloc = pa.Allocator(NB, 16)
    alloc.create(0, 31)                       # 2 blocks; the next token stays in block 1
    alloc.create(1, 32)                       # 2 full blocks; the next token needs a third
    free0 = alloc.num_free()
    tab0 = alloc.block_tables([0, 1], 2)
    buf = np.zeros(pa.pa_decode_step_staging_bytes(2, 4), np.uint8)
    with pytest.raises(pa.PAError) as e:      # unknown sequence (checked before any append)
        pa.pa_decode_step_stage(alloc, [0, 7], 4, buf)
    assert e.value.status == pa.PA_ERR_NOT_FOUND
    with pytest.raises(pa.PAError) as e:      # sequence 1 would need a third column
        pa.pa_decode_step_stage(alloc, [0, 1], 2, buf[:pa.pa_decode_step_staging_bytes(2, 2)])
    assert e.value.status == pa.PA_ERR_INVALID
    with pytest.raises(pa.PAError) as e:      # staging smaller than the bound for 4 columns
        pa.pa_decode_step_stage(alloc, [0, 1], 4, buf[:-1])
    assert e.value.status == pa.PA_ERR_INVALID
    with pytest.raises(pa.PAError) as e:      # misaligned staging
        pa.pa_decode_step_stage(alloc, [0, 1], 4, buf[1:])
    assert e.value.status == pa.PA_ERR_INVALID
    assert alloc.num_free() == free0
    assert np.array_equal(alloc.block_tables([0, 1], 2), tab0)
    assert [alloc.num_tokens(0), alloc.num_tokens(1)] == [31, 32]
    ncow, mx, cols, used = pa.pa_decode_step_stage(alloc, [0, 1], 4, buf)
    assert (ncow, mx, cols) == (0, 33, 3) and alloc.num_free() == free0 - 1


def test_decode_step_argument_checks(pa):
    """Errors that pa_decode_step reports before the allocator changes.  The device
    pointers are fake 256-aligned addresses: no case reaches a HIP call."""
    from paged_kv_cache_57_amd._binding import _lib
    alloc = pa.Allocator(64, 16)
    alloc.create(0, 20)
    ids = np.array([0], np.int64)
    host = np.zeros(pa.pa_decode_step_staging_bytes(1, 8), np.uint8)
    fake = ctypes.c_void_p(1 << 20)
    H, d = 4, 64
    ws_need = pa.pa_forward_workspace_bytes(1, 1, 1, H, H, d, 16 * 8, pa.PA_BF16)

    def call(out=fake, ws=fake, ws_bytes=ws_need, dtype=pa.PA_BF16, head_dim=d, groups=None, ng=0, mbps=8,
             dev_staging=fake, scale=0.125, hq=H, hkv=H):
        return _lib.pa_decode_step(alloc._h, 1, ids.ctypes.data_as(ctypes.c_void_p), None, out, fake, fake, fake, fake,
                                   fake, 64, hq, hkv, head_dim, dtype, scale, groups, ng, mbps,
                                   host.ctypes.data_as(ctypes.c_void_p), dev_staging, host.nbytes, ws, ws_bytes,
                                   None, None)
    assert call(out=None) == pa.PA_ERR_INVALID
    assert call(ws=ctypes.c_void_p((1 << 20) + 64)) == pa.PA_ERR_INVALID          # workspace alignment
    assert call(dev_staging=ctypes.c_void_p((1 << 20) + 4)) == pa.PA_ERR_INVALID  # staging alignment
    assert call(ws_bytes=ws_need - 1) == pa.PA_ERR_INVALID
    assert call(dtype=7) == pa.PA_ERR_UNSUPPORTED
    assert call(head_dim=96) == pa.PA_ERR_UNSUPPORTED
    assert call(dtype=pa.PA_F32, groups=fake, ng=1) == pa.PA_ERR_UNSUPPORTED                  # groups need bf16
    assert call(ng=1) == pa.PA_ERR_INVALID                                         # groups NULL
    assert call(hq=6, hkv=4) == pa.PA_ERR_INVALID
    assert call(scale=float("nan")) == pa.PA_ERR_INVALID
    assert call(mbps=0) == pa.PA_ERR_INVALID
    assert "workspace" in pa.pa_last_error() or "table" in pa.pa_last_error()
    assert alloc.num_tokens(0) == 20 and alloc.num_free() == 62


def test_stage_with_streaming_sequences(pa):
    """Two streaming sequences (4 sinks + a window of 40, one of them forked) beside a
    plain one: once a stream's cache is full, the staged slot is the ring position of
    the mirror, the staged length stays at 44 and a shared block is copied on write."""
    NB = 64
    alloc = pa.Allocator(NB, 16)
    mirror = mirror_alloc.StreamingAllocator(NB, 16)
    alloc.create_streaming(0, 4, 40, 30)
    mirror.create_streaming(0, 4, 40, 30)
    alloc.fork(0, 1)
    mirror.fork(0, 1)
    alloc.create(2, 5)
    mirror.create(2, 5)
    ids = [0, 1, 2]
    M = 8
    buf = np.zeros(pa.pa_decode_step_staging_bytes(len(ids), M), np.uint8)
    cows = 0
    for step in range(60):
        ncow, mx, cols, used = pa.pa_decode_step_stage(alloc, ids, M, buf)
        want_slots, want_pairs = [], []
        for s in ids:
            sl, cow = mirror.append_streaming(s) if s in mirror.stream else mirror.append_slot(s)
            want_slots.append(sl)
            if cow:
                want_pairs.append(cow)
        o_lens, o_qsl, o_pairs, o_tab, end = layout(len(ids), cols)
        assert list(buf[:o_lens].view(np.int64)) == want_slots, step
        assert [tuple(x) for x in buf[o_pairs:o_pairs + 8 * ncow].view(np.int32).reshape(-1, 2)] == want_pairs, step
        lens = [mirror.ntok[s] for s in ids]
        assert list(buf[o_lens:o_qsl].view(np.int32)) == lens, step
        cows += ncow
    assert lens[:2] == [44, 44] and lens[2] == 65 and cows > 0


def test_stage_with_prefix_cached_sequences(pa):
    """Sequences made from token ids (prefix caching on): the step appends each new token
    through pa_seq_append_tokens.  Three requests share a 2-block prompt prefix; the staged
    slots, copy pairs, lengths and tables equal the prefix-caching mirror's every step,
    including the steps where a filled block is registered or replaced by a cached one."""
    NB, P = 64, 16
    rng = np.random.default_rng(4)
    alloc = pa.Allocator(NB, P)
    alloc.enable_prefix_caching()
    mirror = mirror_alloc.PrefixCachingAllocator(NB, P)
    prompt = list(rng.integers(0, 1000, size=2 * P + 5))
    for s in (0, 1, 2):
        toks = prompt if s < 2 else prompt[:2 * P] + [7, 7, 7]
        assert alloc.create_tokens(s, toks) == mirror.create_tokens(s, toks)
    ids = [0, 1, 2]
    switched = 0
    M = 8
    buf = np.zeros(pa.pa_decode_step_staging_bytes(len(ids), M), np.uint8)
    for step in range(40):
        t01, t2 = (int(x) for x in rng.integers(0, 3, size=2))
        new = [t01, t01, t2]              # sequences 0 and 1 fill equal blocks: the second switches to the first's
        before = [list(mirror.block_table(s)) for s in ids]
        ncow, mx, cols, used = pa.pa_decode_step_stage(alloc, ids, M, buf, token_ids=new)
        want_slots, want_pairs = [], []
        for s, tkn in zip(ids, new):
            sl, cow = mirror.append_token(s, tkn)
            want_slots.append(sl)
            if cow:
                want_pairs.append(cow)
        o_lens, o_qsl, o_pairs, o_tab, end = layout(len(ids), cols)
        assert list(buf[:o_lens].view(np.int64)) == want_slots, step
        assert [tuple(x) for x in buf[o_pairs:o_pairs + 8 * ncow].view(np.int32).reshape(-1, 2)] == want_pairs
        assert list(buf[o_lens:o_qsl].view(np.int32)) == [mirror.ntok[s] for s in ids], step
        want_tab = np.full((len(ids), cols), -1, np.int32)
        for i, s in enumerate(ids):
            t = mirror.block_table(s)
            want_tab[i, :len(t)] = t
        assert np.array_equal(buf[o_tab:end].view(np.int32).reshape(len(ids), cols), want_tab), step
        assert alloc.num_free() == mirror.num_free()
        switched += sum(1 for i, s in enumerate(ids)
                        if len(before[i]) == len(mirror.block_table(s)) and before[i] != list(mirror.block_table(s)))
    assert switched > 0
    with pytest.raises(pa.PAError) as e:                       # a token per sequence
        pa.pa_decode_step_stage(alloc, ids, M, buf, token_ids=[1])
    assert e.value.status == pa.PA_ERR_INVALID
    with pytest.raises(pa.PAError):                            # these sequences take token ids
        pa.pa_decode_step_stage(alloc, ids, M, buf)
