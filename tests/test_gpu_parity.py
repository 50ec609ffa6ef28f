"""GPU parity of libpa against the fp64 CPU oracle (MI355X, through the C ABI)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import cache_ops
from tests._gpu import (DEV, Run, assert_close, check_tables_in_pool, host_raw, oracle_rows, oracle_rows_all,
                        say, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_57_amd as pa
    assert torch.cuda.is_available()
    return pa


def run_and_check(pa, w, seqs=None, poison=False, label=None):
    """Draw the workload's values, run (cache write +) forward, compare every row of the
    listed sequences (default: all of them) with the oracle."""
    label = label or w.name
    say(f"[case] {label}: S={w.num_seqs} T={w.num_tokens} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"d={w.head_dim} {w.dtype} NB={w.num_blocks} maxL={w.max_context_len}")
    check_tables_in_pool(w)
    r = Run(w)
    q, kc, vc, nk, nv = W.make_values(w, DEV)
    if poison:
        poison_unreferenced(w, kc, vc)
    if nk is not None:
        r.write(nk, nv, kc, vc)
    out = r.forward(q, kc, vc)
    r.check_status()
    rows, ref = oracle_rows_all(w, q, kc, vc, seqs)
    got = to_f64(out.index_select(0, torch.from_numpy(rows).to(DEV)))
    assert np.isfinite(got).all()
    assert_close(got, ref, w.dtype, label)
    return out, (q, kc, vc), r


def poison_unreferenced(w, kc, vc):
    """NaN in every block no table references and in the unused tail slots of last blocks."""
    used = np.zeros(w.num_blocks, bool)
    for s, L in enumerate(w.context_lens):
        n = (int(L) + 15) // 16
        used[w.block_tables[s, :n]] = True
        if L % 16:
            b = int(w.block_tables[s, n - 1])
            kc[b, :, :, L % 16:, :] = float("nan")
            vc[b, :, :, L % 16:] = float("nan")
    free = torch.from_numpy(np.flatnonzero(~used)).to(DEV)
    if free.numel():
        kc[free] = float("nan")
        vc[free] = float("nan")


# ---------------------------------------------------------------- cache write and copy

@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_reshape_and_cache_bit_exact(pa, dtype, d):
    say(f"[case] reshape_and_cache {dtype} d={d}")
    rng = np.random.default_rng(d)
    nb, hkv, T = 37, 3, 300
    run = np.arange(160, 200)                                # a run of consecutive slots
    rest = np.setdiff1d(rng.permutation(nb * 16), run)
    slots = np.concatenate([run, rng.permutation(rest)[:T - run.size]]).astype(np.int64)
    slots[[5, 77, 250]] = -1                                 # padding tokens
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    ks, vs = W.cache_shapes(nb, hkv, d, dtype)
    g = torch.Generator(device=DEV).manual_seed(1)
    kc = W.fill_normal(torch.empty(ks, dtype=td, device=DEV), g)
    vc = W.fill_normal(torch.empty(vs, dtype=td, device=DEV), g)
    key = W.fill_normal(torch.empty((T, hkv, d), dtype=td, device=DEV), g)
    val = W.fill_normal(torch.empty((T, hkv, d), dtype=td, device=DEV), g)
    k0, v0 = host_raw(kc), host_raw(vc)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    pa.pa_reshape_and_cache(key, val, kc, vc, torch.from_numpy(slots).to(DEV), st)
    torch.cuda.synchronize()
    assert st.item() == 0
    k1, v1 = cache_ops.reshape_and_cache(host_raw(key), host_raw(val), k0, v0, slots)
    assert np.array_equal(host_raw(kc).view(np.uint8), k1.view(np.uint8))
    assert np.array_equal(host_raw(vc).view(np.uint8), v1.view(np.uint8))


def test_copy_blocks_bit_exact(pa):
    say("[case] copy_blocks bf16 d=128 Hkv=32")
    nb, hkv, d = 24, 32, 128
    ks, vs = W.cache_shapes(nb, hkv, d, "bf16")
    g = torch.Generator(device=DEV).manual_seed(2)
    kc = W.fill_normal(torch.empty(ks, dtype=torch.bfloat16, device=DEV), g)
    vc = W.fill_normal(torch.empty(vs, dtype=torch.bfloat16, device=DEV), g)
    pairs = np.array([[3, 10], [3, 11], [7, 0], [23, 12]], np.int32)
    k0, v0 = host_raw(kc), host_raw(vc)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    pa.pa_copy_blocks(kc, vc, torch.from_numpy(pairs).to(DEV), st)
    torch.cuda.synchronize()
    assert st.item() == 0
    k1, v1 = cache_ops.copy_blocks(k0, v0, pairs)
    assert np.array_equal(host_raw(kc), k1) and np.array_equal(host_raw(vc), v1)


def test_out_of_range_ids_are_flagged_not_followed(pa):
    # the kernels check ids before forming an address; the host sees the status bits
    say("[case] out-of-range slot / pair / table entry")
    nb, hkv, d = 4, 1, 64
    ks, vs = W.cache_shapes(nb, hkv, d, "f32")
    kc = torch.zeros(ks, device=DEV)
    vc = torch.zeros(vs, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    key = torch.ones((2, hkv, d), device=DEV)
    pa.pa_reshape_and_cache(key, key, kc, vc, torch.tensor([3, nb * 16], device=DEV), st)
    pa.pa_copy_blocks(kc, vc, torch.tensor([[0, 1], [2, nb]], dtype=torch.int32, device=DEV), st)
    torch.cuda.synchronize()
    assert st.item() == pa.PA_DEV_BAD_SLOT | pa.PA_DEV_BAD_BLOCK
    w = W.random_ragged(0, "f32", 2, 2, 64, [1], [20])
    w.block_tables[0, 1] = w.num_blocks + 5                 # second page points outside the pool
    r = Run(w)
    q, kc2, vc2, _, _ = W.make_values(w, DEV)
    r.forward(q, kc2, vc2)
    torch.cuda.synchronize()
    assert r.status.item() == pa.PA_DEV_BAD_BLOCK


# ---------------------------------------------------------------- attention parity

def test_tiny_decode_fp32(pa):
    run_and_check(pa, W.tiny_decode(0))


# Case 1 (float32, head_dim 128) faulted the GPU on the first run and case 2
# hung on the second.  Cause, read from the generated code: the work loop
# fetched items with "lane 0 takes an atomic ticket, readfirstlane shares it",
# and the compiler merged that lane-0 branch with the lane-0 store at the end
# of an item, leaving lanes 1..63 in an inner loop with a stale item (a hang)
# and reading a block id from the inactive lane 0 (the fault).  The workers now
# have no per-lane branches (checked on the compiled code by
# test_kernel_resources), and both cases run.
REJECTED = {}  # cases the host refuses (index -> message); none at present

RAGGED = [
    # dtype, Hq, Hkv, d, q_lens, ctx_lens
    ("f32", 4, 4, 64, [1, 1, 1], [1, 16, 17]),
    ("f32", 8, 2, 128, [1, 5, 1], [1300, 40, 513]),              # float32 at head_dim 128: VALU rows, GQA, prefill
    ("f32", 8, 2, 64, [1, 5, 1], [1300, 40, 513]),               # VALU split contexts, GQA, fp32 prefill rows
    ("bf16", 32, 32, 128, [1, 1, 1, 1], [1, 15, 513, 2049]),      # MHA decode, partitions + ragged tails
    ("bf16", 8, 8, 64, [1, 1], [700, 33]),
    ("bf16", 64, 8, 128, [1, 1, 1], [1, 255, 1000]),              # GQA decode, 256-key partitions
    ("bf16", 16, 2, 64, [1, 1], [300, 17]),
    ("bf16", 8, 8, 128, [37, 1, 16, 1], [37, 900, 1100, 2]),      # prefill tiles (prior 0 and 1084)
    ("bf16", 16, 4, 128, [9, 3, 1], [2100, 3, 64]),               # GQA prefill: rows = positions x heads
    ("bf16", 4, 4, 64, [70, 1], [1500, 5]),                       # prefill crossing partitions of 1024
    ("bf16", 2, 2, 128, [300, 1], [2500, 40]),                    # 128-row tiles: 3 tiles, last one 44 rows
    ("bf16", 16, 2, 64, [40, 17], [40, 1100]),                    # GQA tiles: 320 and 136 rows
    ("bf16", 4, 4, 128, [129, 128, 2], [129, 1152, 2]),           # tile edges: 129 and 128 rows, 2-row MFMA
    ("bf16", 2, 2, 64, [1, 3], [33000, 700]),                     # >= 32 partitions: four waves merge a row
    ("f32", 2, 2, 64, [1, 2], [33500, 40]),                       # the same for float32 (1024-key partitions)
    ("f32", 4, 4, 128, [1, 3], [9000, 130]),                      # float32 at head_dim 128: 9 partitions merged
    ("bf16", 2, 2, 128, [1, 1, 2], [20000, 9000, 100]),           # 20 and 9 partitions: one wavefront, load rounds
]


@pytest.mark.parametrize("i", range(len(RAGGED)))
def test_ragged_batches(pa, i):
    dt, hq, hkv, d, ql, cl = RAGGED[i]
    w = W.random_ragged(100 + i, dt, hq, hkv, d, ql, cl)
    if i in REJECTED:                       # refused on the host, nothing is launched
        r = Run(w)
        q = torch.zeros((w.num_tokens, hq, d), device=DEV)
        ks, vs = W.cache_shapes(w)
        with pytest.raises(pa.PAError) as e:
            r.forward(q, torch.zeros(ks, device=DEV), torch.zeros(vs, device=DEV))
        assert e.value.status == pa.PA_ERR_UNSUPPORTED and REJECTED[i] in str(e.value)
        return
    run_and_check(pa, w, label=f"ragged[{i}] {dt} Hq={hq} Hkv={hkv} d={d} q={ql} L={cl}")


DEGENERATE = [
    # dtype, Hq, Hkv, d, q_lens, ctx_lens
    ("bf16", 16, 2, 64, [0, 1, 0, 5, 0, 1], [0, 300, 17, 40, 0, 1]),    # idle slots (no keys, no rows) among live ones
    ("f32", 4, 4, 128, [0, 2, 0], [0, 1500, 0]),                        # float32, one live sequence between idle slots
    ("bf16", 4, 4, 64, [0, 32, 16, 0], [0, 32, 1024, 2048]),            # whole prompt from position 0, block-aligned lengths
]


@pytest.mark.parametrize("i", range(len(DEGENERATE)))
def test_idle_slots_and_block_aligned_lengths(pa, i):
    # sequences with no query rows (with or without keys) must neither be read nor written;
    # unreferenced pages hold NaN so a stray read shows up in the live rows
    dt, hq, hkv, d, ql, cl = DEGENERATE[i]
    w = W.random_ragged(300 + i, dt, hq, hkv, d, ql, cl)
    run_and_check(pa, w, poison=True, label=f"degenerate[{i}] {dt} q={ql} L={cl}")


def test_batches_without_query_rows(pa):
    # no rows (every sequence idle) and no sequences at all: the call succeeds, launches
    # nothing and leaves the status word alone
    w = W.random_ragged(310, "bf16", 8, 8, 128, [0, 0, 0], [0, 64, 0])
    r = Run(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    assert q.shape[0] == 0
    out = r.forward(q, kc, vc)
    r.check_status()
    assert out.shape == (0, 8, 128)
    i32 = dict(dtype=torch.int32, device=DEV)
    st = torch.full((1,), 0, **i32)
    empty_q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=DEV)
    pa.pa_forward(torch.empty_like(empty_q), empty_q, kc, vc, torch.empty((0, 1), **i32), torch.empty(0, **i32),
                  torch.zeros(1, **i32), 0, 0, w.scale, r.workspace, st)
    pa.pa_reshape_and_cache(torch.empty((0, 8, 128), dtype=torch.bfloat16, device=DEV),
                            torch.empty((0, 8, 128), dtype=torch.bfloat16, device=DEV), kc, vc,
                            torch.empty(0, dtype=torch.int64, device=DEV), st)
    before = host_raw(kc).copy()
    pa.pa_copy_blocks(kc, vc, torch.empty((0, 2), **i32), st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(host_raw(kc), before)


def random_batch(seed, max_seqs=10, max_ctx=3000, max_chunk=300):
    """A seeded random mixed batch: dtype, head dimension, query heads per KV head and a mix
    of idle sequences, decodes and prefill chunks (prior context 0 .. max_ctx)."""
    rng = np.random.default_rng(1000 + seed)
    dt = "f32" if rng.random() < 0.25 else "bf16"
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    n = int(rng.integers(1, max_seqs + 1))
    kind = rng.choice(["idle", "decode", "chunk"], size=n, p=[0.1, 0.55, 0.35])
    ql = np.where(kind == "idle", 0, np.where(kind == "decode", 1, rng.integers(2, max_chunk + 1, size=n)))
    cl = ql + rng.integers(0, max_ctx + 1, size=n)
    cl[kind == "idle"] = rng.integers(0, 50, size=int((kind == "idle").sum()))
    return W.random_ragged(2000 + seed, dt, G * hkv, hkv, d, [int(x) for x in ql], [int(x) for x in cl])


def many_sequences_batch(n=5000, n_split=12, split_hi=1500, heads=2):
    """n sequences (more than the 2,047 the workers' LDS lookup table holds one by one):
    MHA decodes, some split into partitions, plus short prefill rows and empty-query sequences."""
    rng = np.random.default_rng(31)
    ql = np.ones(n, np.int64)
    ql[rng.choice(n, 40, replace=False)] = 0                  # sequences with no query rows this pass
    ql[rng.choice(n, 20, replace=False)] = 3                  # short prefill rows (MFMA class)
    cl = rng.integers(1, 90, size=n)
    cl[rng.choice(n, n_split, replace=False)] = rng.integers(600, split_hi, size=n_split)   # split contexts
    cl = np.maximum(cl, ql)
    return W.random_ragged(32, "bf16", heads, heads, 64, ql, cl)


def shared_prefix_batch(seed, hq, hkv, d, groups_spec, loose_decodes=2, chunk=(5, 300), bad_group=False):
    """A batch whose decode sequences come in groups sharing the pages of a prompt.
    groups_spec: [(members, prompt length)]; every member's context is the prompt plus a
    few tokens of its own (its own partial and later pages), and the group shares the
    prompt's full pages (shared keys = 16 * floor(prompt / 16)).  Plus loose decodes and
    one prefill chunk (q_len, context) that belong to no group.  With bad_group the last
    group's second member gets a different page at position 0 (the group must be refused).
    Returns the workload and the [G, 3] group list."""
    rng = np.random.default_rng(seed)
    lens, qls, tabs, groups = [], [], [], []
    nxt = [0]
    def fresh(n):
        ids = list(range(nxt[0], nxt[0] + n))
        nxt[0] += n
        return ids
    for members, plen in groups_spec:
        shared = fresh(plen // 16)
        groups.append([len(lens), members, 16 * (plen // 16)])
        for m in range(members):
            L = plen + int(rng.integers(1, 40))
            own = fresh((L + 15) // 16 - len(shared))
            lens.append(L)
            qls.append(1)
            tabs.append(shared + own)
    for _ in range(loose_decodes):
        L = int(rng.integers(20, 700))
        lens.append(L)
        qls.append(1)
        tabs.append(fresh((L + 15) // 16))
    if chunk:
        q, L = chunk
        lens.append(L)
        qls.append(q)
        tabs.append(fresh((L + 15) // 16))
    if bad_group:
        g = groups[-1]
        tabs[g[0] + 1] = [fresh(1)[0]] + tabs[g[0] + 1][1:]
    nb = nxt[0] + 4
    perm = rng.permutation(nb).astype(np.int32)          # physical blocks in random order
    mb = max(len(t) for t in tabs)
    tables = np.full((len(lens), mb), -1, np.int32)
    for i, t in enumerate(tabs):
        tables[i, :len(t)] = perm[np.asarray(t)]
    qsl = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    w = W.Workload(f"shared_s{seed}", "bf16", hq, hkv, d, nb, np.asarray(lens, np.int32), qsl, tables,
                   float(np.float32(1.0 / np.sqrt(d))), None, seed)
    return w, np.asarray(groups, np.int32)


SHARED_CASES = [  # (seed, hq, hkv, d, groups, bad)
    (1, 8, 8, 128, [(3, 100), (4, 530), (2, 40)], False),
    (2, 8, 2, 128, [(4, 300), (2, 1100)], False),
    (3, 4, 4, 64, [(16, 70), (3, 2100)], False),
    (4, 8, 8, 128, [(3, 100), (2, 200)], True),
]


@pytest.mark.parametrize("seed", range(24))
def test_random_batches(pa, seed):
    # every row of a seeded random batch against the oracle, unreferenced pages poisoned
    w = random_batch(seed)
    run_and_check(pa, w, poison=True, label=f"random[{seed}] {w.dtype} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
                                             f"d={w.head_dim} q={list(np.diff(w.query_start_loc))} "
                                             f"L={list(w.context_lens)}")


def test_many_sequences(pa):
    w = many_sequences_batch()
    run_and_check(pa, w, label="5000 sequences")


def test_length_order_over_many_sequences(pa):
    # 1500 one-head decode sequences: few VALU items per resident wavefront, so the planner
    # sorts the last partitions by length, over two chunks of 1024 sequences in both passes
    rng = np.random.default_rng(33)
    cl = rng.integers(1, 3000, size=1500)
    w = W.random_ragged(33, "bf16", 1, 1, 128, [1] * len(cl), [int(x) for x in cl])
    run_and_check(pa, w, label="length order, 1500 sequences")


def test_very_long_contexts(pa):
    """Contexts of 131,072 keys: 256 VALU partitions (MHA decode, bf16 and float32) and
    512 MFMA partitions (GQA decode) merged per row, plus a 130-row prefill chunk at the
    end of a 40,000-key context (40 tile partitions per row, two row tiles)."""
    for dt, hq, hkv, d, ql, cl in [("bf16", 2, 2, 128, [1, 1], [131072, 5]),
                                   ("f32", 2, 2, 64, [1], [131072]),
                                   ("bf16", 16, 2, 128, [1, 1], [131072, 700]),
                                   ("bf16", 2, 2, 128, [130], [40000])]:
        w = W.random_ragged(77, dt, hq, hkv, d, ql, cl)
        run_and_check(pa, w, label=f"long {dt} Hq={hq} Hkv={hkv} d={d} q={ql} L={cl}")


def test_nan_poison_outside_context(pa):
    w = W.random_ragged(7, "bf16", 16, 4, 128, [1, 5, 1, 1], [37, 600, 1000, 1])
    run_and_check(pa, w, poison=True, label="nan-poison GQA")
    w = W.random_ragged(8, "bf16", 8, 8, 128, [1, 1, 20], [517, 33, 1025])
    run_and_check(pa, w, poison=True, label="nan-poison MHA")


# Scales other than 1/sqrt(d): negative (the tile worker flips the sign of q),
# zero (every visible key weighs the same) and large (sharp weights).
SCALES = [-0.0625, 0.0, 0.75]


@pytest.mark.parametrize("scale", SCALES)
def test_scale_sign_and_size(pa, scale):
    # decode rows (VALU), GQA rows (MFMA) and a 128-row prefill tile (TILE) in two batches
    for hq, hkv, ql, cl in [(8, 8, [1, 150, 1], [700, 1200, 40]), (16, 4, [1, 40], [300, 1100])]:
        w = W.random_ragged(20, "bf16", hq, hkv, 128, ql, cl)
        w.scale = float(np.float32(scale))
        run_and_check(pa, w, label=f"scale {scale} Hq={hq} Hkv={hkv} q={ql} L={cl}")


@pytest.mark.parametrize("k", [20, 24, 30])
def test_large_value_magnitudes(pa, k):
    # values scaled by 2^k: the prefill tile stages values as half when every staged
    # magnitude is below 2^16 and recomputes an item in bfloat16 (weights split in a high
    # and a low part) when one is not; every worker stays within tolerance, never NaN
    w = W.random_ragged(21, "bf16", 8, 8, 128, [1, 150, 1], [700, 1200, 40])
    say(f"[case] large value magnitudes (V x 2^{k}, K x 4)")
    r = Run(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    vc.mul_(2.0 ** k)
    kc.mul_(4.0)
    out = r.forward(q, kc, vc)
    r.check_status()
    rows, ref = oracle_rows_all(w, q, kc, vc)
    got = to_f64(out.index_select(0, torch.from_numpy(rows).to(DEV)))
    assert np.isfinite(got).all()
    # the output scales with the values (an exact power of two): compare at the scale of N(0, 1) values
    assert_close(got / 2.0 ** k, ref / 2.0 ** k, "bf16", f"large value magnitudes (/2^{k})")


def test_huge_value_on_a_causally_masked_key(pa):
    # one key inside a prefill chunk holds values of 2^30: the rows before it must not see it
    # (no 0 x inf in the P.V of a step), the rows after it weigh it exactly
    for hq, hkv, ql, cl, pos in [(4, 4, [200], [200], 5), (16, 4, [1, 90], [300, 700], 650)]:
        w = W.random_ragged(24, "bf16", hq, hkv, 128, ql, cl)
        say(f"[case] 2^30 on key {pos}: Hq={hq} Hkv={hkv} q={ql} L={cl}")
        r = Run(w)
        q, kc, vc, _, _ = W.make_values(w, DEV)
        s = len(ql) - 1
        b = int(w.block_tables[s, pos // 16])
        vc[b, :, :, pos % 16] = 2.0 ** 30
        out = r.forward(q, kc, vc)
        r.check_status()
        rows, ref = oracle_rows_all(w, q, kc, vc)
        got = to_f64(out.index_select(0, torch.from_numpy(rows).to(DEV)))
        assert np.isfinite(got).all()
        assert_close(got, ref, "bf16", f"2^30 at key {pos}")


def test_score_jump_after_the_first_step(pa):
    # one key's vector scaled by 2^6 (exact in bfloat16): its scores jump far above the
    # maximum of the prefill item's first step; the item's half weights overflow and it is
    # computed again by the exact pass.  Rows before the key must not see it.
    # A GQA decode batch (the one-pass kernel) with a key scaled by 2^10: a jump past 2^127 in
    # the weights of the wavefront that holds it, which is computed again with a row maximum
    # on every step.
    for hq, hkv, ql, cl, pos, k in [(4, 4, [40], [40], 35, 6), (8, 2, [1, 300], [90, 1500], 1300, 6),
                                    (32, 32, [512], [2000], 1900, 6), (64, 8, [1, 1], [32768, 700], 30000, 10),
                                    (16, 2, [1, 1], [3000, 700], 2500, 10)]:
        say(f"[case] key {pos} x 2^{k} Hq={hq} Hkv={hkv} q={ql} L={cl}")
        w = W.random_ragged(26, "bf16", hq, hkv, 128, ql, cl)
        r = Run(w)
        q, kc, vc, _, _ = W.make_values(w, DEV)
        b = int(w.block_tables[len(ql) - 1, pos // 16])
        kc[b, :, :, pos % 16] *= 2.0 ** k
        out = r.forward(q, kc, vc)
        r.check_status()
        rows, ref = oracle_rows_all(w, q, kc, vc)
        got = to_f64(out.index_select(0, torch.from_numpy(rows).to(DEV)))
        assert np.isfinite(got).all()
        assert_close(got, ref, "bf16", f"key {pos} x 2^{k}")


def test_single_key_and_equal_scores(pa):
    # one key: output is that value row exactly; q = 0: output is the mean of the values
    for dt, hq, hkv, d in [("f32", 4, 4, 64), ("bf16", 32, 32, 128), ("bf16", 64, 8, 128)]:
        say(f"[case] single key / equal scores {dt} Hq={hq} Hkv={hkv}")
        w = W.random_ragged(9, dt, hq, hkv, d, [1, 1], [1, 1])
        r = Run(w)
        q, kc, vc, _, _ = W.make_values(w, DEV)
        out = r.forward(q, kc, vc)
        r.check_status()
        for s in range(2):
            b = int(w.block_tables[s, 0])
            v = to_f64(vc[b, :, :, 0])                         # [Hkv, d]
            got = to_f64(out[s]).reshape(hkv, hq // hkv, -1)
            assert np.array_equal(got, np.repeat(v[:, None], hq // hkv, 1))
    w = W.random_ragged(10, "bf16", 32, 32, 128, [1], [777])
    r = Run(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    q.zero_()
    out = r.forward(q, kc, vc)
    r.check_status()
    rows, ref = oracle_rows(w, q, kc, vc, [0])
    assert_close(to_f64(out), ref, "bf16", "q=0 mean of values")


def test_block_permutation_gives_identical_bits(pa):
    w = W.random_ragged(11, "bf16", 16, 2, 128, [1, 7, 1], [900, 300, 47])
    say("[case] physical block permutation (bit-identical)")
    r = Run(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    base = r.forward(q, kc, vc).clone()
    perm = np.random.default_rng(5).permutation(w.num_blocks)
    kc2, vc2 = torch.empty_like(kc), torch.empty_like(vc)
    pt = torch.from_numpy(perm).to(DEV)
    kc2[pt] = kc
    vc2[pt] = vc
    w2 = W.Workload(**{**w.__dict__})
    w2.block_tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    r2 = Run(w2)
    out2 = r2.forward(q, kc2, vc2)
    r2.check_status()
    assert torch.equal(base.view(torch.int16), out2.view(torch.int16))


def test_batch_invariance(pa):
    # a sequence's output is bit-identical alone and inside a bigger batch
    say("[case] batch invariance")
    w = W.random_ragged(12, "bf16", 32, 32, 128, [1, 1, 1, 1], [2049, 100, 3000, 512])
    r = Run(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    full = r.forward(q, kc, vc).clone()
    for s in range(w.num_seqs):
        ws = W.Workload(**{**w.__dict__})
        ws.context_lens = w.context_lens[s:s + 1].copy()
        ws.block_tables = w.block_tables[s:s + 1].copy()
        ws.query_start_loc = np.array([0, 1], np.int32)
        rs = Run(ws)
        one = rs.forward(q[s:s + 1].contiguous(), kc, vc)
        rs.check_status()
        assert torch.equal(one.view(torch.int16), full[s:s + 1].view(torch.int16)), s


def test_item_order_does_not_change_results(pa):
    # A batch in which neighbouring sequences share pages walks the VALU items in a fixed
    # strided order with plain page loads; a batch without takes them by ticket with
    # non-temporal loads.  A sequence's output is bit-identical either way.
    w = W.random_ragged(14, "bf16", 32, 32, 128, [1, 1, 1, 1], [2049, 3000, 3000, 700])
    w.block_tables[2, :] = w.block_tables[1, :]  # sequences 1 and 2 read the same pages
    say("[case] VALU item order: strided (shared pages) vs tickets (alone)")
    check_tables_in_pool(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    r = Run(w)
    full = r.forward(q, kc, vc).clone()
    r.check_status()
    rows, ref = oracle_rows_all(w, q, kc, vc)
    assert_close(to_f64(full.index_select(0, torch.from_numpy(rows).to(DEV))), ref, "bf16", "strided VALU order")
    for s in range(w.num_seqs):
        ws = W.Workload(**{**w.__dict__})
        ws.context_lens = w.context_lens[s:s + 1].copy()
        ws.block_tables = w.block_tables[s:s + 1].copy()
        ws.query_start_loc = np.array([0, 1], np.int32)
        rs = Run(ws)
        one = rs.forward(q[s:s + 1].contiguous(), kc, vc)
        rs.check_status()
        assert torch.equal(one.view(torch.int16), full[s:s + 1].view(torch.int16)), s


def test_batch_invariance_gqa_decode(pa):
    # decode-only GQA batches take the one-pass kernel: a sequence's output is bit-identical
    # alone and inside a bigger batch (partition lengths follow the sequence's own length)
    say("[case] batch invariance, one-pass GQA decode")
    w = W.random_ragged(13, "bf16", 64, 8, 128, [1, 1, 1, 1], [9000, 100, 3000, 2049])
    r = Run(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    full = r.forward(q, kc, vc).clone()
    r.check_status()
    rows, ref = oracle_rows_all(w, q, kc, vc)
    assert_close(to_f64(full.index_select(0, torch.from_numpy(rows).to(DEV))), ref, "bf16", "one-pass GQA decode")
    for s in range(w.num_seqs):
        ws = W.Workload(**{**w.__dict__})
        ws.context_lens = w.context_lens[s:s + 1].copy()
        ws.block_tables = w.block_tables[s:s + 1].copy()
        ws.query_start_loc = np.array([0, 1], np.int32)
        rs = Run(ws)
        one = rs.forward(q[s:s + 1].contiguous(), kc, vc)
        rs.check_status()
        assert torch.equal(one.view(torch.int16), full[s:s + 1].view(torch.int16)), s


def test_gqa_decode_replayed_from_a_hip_graph(pa):
    """The one-pass GQA decode (tagged completion counters in the workspace, left at zero by
    the merging workgroup) captured once and replayed with new inputs: every replay equals
    the eager call bit for bit, and the oracle on the last one."""
    w = W.random_ragged(42, "bf16", 64, 8, 128, [1, 1, 1], [9000, 5000, 1500], with_slots=True)
    say(f"[case] HIP graph replay of the one-pass GQA decode: L={list(w.context_lens)}")
    check_tables_in_pool(w)
    q, kc, vc, nk, nv = W.make_values(w, DEV)
    r = Run(w)
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r.write(nk, nv, kc, vc)
        r.forward(q, kc, vc, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.write(nk, nv, kc, vc)
        r.forward(q, kc, vc, out)
    gen = torch.Generator(device=DEV).manual_seed(4)
    for rep in range(4):
        W.fill_normal(q, gen)
        W.fill_normal(nk, gen)
        W.fill_normal(nv, gen)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        r.write(nk, nv, kc, vc)
        ref_out = r.forward(q, kc, vc)
        r.check_status()
        assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep} differs"
    rows, ref = oracle_rows_all(w, q, kc, vc)
    assert_close(to_f64(got.index_select(0, torch.from_numpy(rows).to(DEV))), ref, "bf16", "graph replay, one-pass")


# ---------------------------------------------------------------- the benchmark workloads

def test_llama7b_decode_batch64(pa):
    run_and_check(pa, W.llama7b_decode(0))


def test_gqa70b_decode_batch32(pa):
    run_and_check(pa, W.gqa70b_decode(0))


def test_gqa70b_decode_long_32k(pa):
    run_and_check(pa, W.gqa70b_long_decode(0))


def test_splitfuse_mixed_pass(pa):
    # every row: both prefill chunks (1024 rows) and all 1024 decode rows, after the cache write
    w = W.splitfuse_mixed(0)
    run_and_check(pa, w)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 2)])
def test_chunk_last_row_equals_decode_row(pa, hq, hkv):
    """The last row of a prefill chunk and a decode query at the same position, over the
    same cache, give the same attention (the prefill tile worker against the decode
    workers: VALU for one query head per KV head, MFMA for GQA), each within tolerance
    of the oracle and of each other."""
    say(f"[case] chunk last row = decode row, Hq={hq} Hkv={hkv}")
    w = W.random_ragged(51, "bf16", hq, hkv, 128, [300, 1], [2900, 700])
    r = Run(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    out = r.forward(q, kc, vc)
    r.check_status()
    last = int(w.query_start_loc[1]) - 1                 # the chunk's last row sits at position L - 1
    wd = W.Workload(**{**w.__dict__})
    wd.context_lens = w.context_lens[:1].copy()
    wd.block_tables = w.block_tables[:1].copy()
    wd.query_start_loc = np.array([0, 1], np.int32)
    rd = Run(wd)
    qd = q[last:last + 1].contiguous()
    outd = rd.forward(qd, kc, vc)
    rd.check_status()
    rows, ref = oracle_rows_all(wd, qd, kc, vc)
    got_chunk, got_dec = to_f64(out[last:last + 1]), to_f64(outd)
    assert_close(got_dec, ref, "bf16", "decode row")
    assert_close(got_chunk, ref, "bf16", "chunk last row")
    assert_close(got_chunk, got_dec, "bf16", "chunk last row vs decode row")


def test_parallel_sampling_workflow(pa):
    # 16 prompts x 4 branches sharing prompt pages, copy-on-write at step 0, 256 decode steps;
    # slots, copy pairs and tables checked every step, pool bytes and outputs at checkpoints
    from tests._sampling import GpuBackend, run_workflow
    spec = W.parallel_sampling_spec(0)
    say(f"[case] parallel sampling: prompts {list(spec.prompt_lens)} x {spec.branches} branches, "
        f"{spec.steps} steps, NB={spec.num_blocks}")
    worst, copies = run_workflow(GpuBackend(pa, spec), spec, checkpoints={0, 1, 15, 16, 17, 255}, say=say)
    say(f"  copy-on-write pairs: {copies}; worst err/bound {worst:.3f}")
    assert copies > 0


def test_composer_driven_passes(pa):
    """Passes composed by the SplitFuse composer (budget 2048, prompts of 3000, 700,
    300 tokens, then 5000 and 64 arriving later) run end to end: allocator slots,
    cache write of every new token, one forward per pass; every row against the
    oracle on a host copy of the pool."""
    from oracle import attention as oattn
    from oracle import cache_ops
    from tests._gpu import TOL, host_raw
    H, d, NB, budget = 8, 128, 2048, 2048
    ks, vs = W.cache_shapes(NB, H, d, "bf16")
    gen = torch.Generator(device=DEV).manual_seed(3)
    kc = W.fill_normal(torch.empty(ks, dtype=torch.bfloat16, device=DEV), gen)
    vc = W.fill_normal(torch.empty(vs, dtype=torch.bfloat16, device=DEV), gen)
    kh, vh = host_raw(kc).copy(), host_raw(vc).copy()
    alloc = pa.Allocator(NB, 16)
    comp = pa.SplitFuse(budget)
    prompts = {0: 3000, 1: 700, 2: 300, 3: 5000, 4: 64}
    arrive = {0: [0, 1, 2], 2: [3, 4]}
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    worst = 0.0
    for step in range(8):
        for sid in arrive.get(step, []):
            comp.add_prompt(sid, prompts[sid])
        ids, ql, cl = comp.step()
        assert int(ql.sum()) <= budget
        slots = []
        for sid, q, ctx in zip(ids.tolist(), ql.tolist(), cl.tolist()):
            if ctx == q:                          # first chunk: pages for the whole prompt
                alloc.create(sid, prompts[sid])
            if ctx <= prompts[sid]:
                slots.append(alloc.slots(sid, ctx - q, q))
            else:
                slot, cow = alloc.append_slot(sid)
                assert cow is None
                slots.append(np.array([slot], np.int64))
        slots = np.concatenate(slots)
        T = len(slots)
        k_new = W.fill_normal(torch.empty((T, H, d), dtype=torch.bfloat16, device=DEV), gen)
        v_new = W.fill_normal(torch.empty((T, H, d), dtype=torch.bfloat16, device=DEV), gen)
        q = W.fill_normal(torch.empty((T, H, d), dtype=torch.bfloat16, device=DEV), gen)
        pa.pa_reshape_and_cache(k_new, v_new, kc, vc, torch.from_numpy(slots).to(DEV), status)
        cache_ops.reshape_and_cache(host_raw(k_new), host_raw(v_new), kh, vh, slots, inplace=True)
        lens = cl.astype(np.int32)
        qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        cap = int((lens.max() + 15) // 16)
        tables = alloc.block_tables(ids, max(cap, max(len(alloc.block_table(int(s))) for s in ids)))
        nbytes = pa.pa_forward_workspace_bytes(len(ids), T, int(ql.max()), H, H, d, int(lens.max()), pa.PA_BF16)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
        out = torch.empty_like(q)
        say(f"[case] composer pass {step}: rows {len(ids)}, tokens {T}, max q {int(ql.max())}, max ctx {int(lens.max())}")
        pa.pa_forward(out, q, kc, vc, torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV),
                      torch.from_numpy(qsl).to(DEV), int(ql.max()), int(lens.max()), scale, ws, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        ref = oattn.paged_attention(host_raw(q), kh, vh, tables, lens, qsl, scale, "bf16")
        got = to_f64(out)
        a, r = TOL["bf16"]
        ratio = float((np.abs(got - ref) / (a + r * np.abs(ref))).max())
        worst = max(worst, ratio)
        assert np.isfinite(got).all() and ratio <= 1.0, (step, ratio)
    say(f"  worst err/bound {worst:.3f}")
    comp.close()
    alloc.close()


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_rope_cache_write(pa, dtype, d):
    """Rotary cache write: rotated q and key against the exact rotation (within the float32
    evaluation's rounding), values and untouched pool bytes bit-exact."""
    from tests import _rope
    from tests._pools import empty_pools, raw
    rng = np.random.default_rng(21)
    T, hq, hkv, nb, maxpos = 300, 32, 8, 64, 8192
    kp, vp = empty_pools(rng, dtype, nb, hkv, d)
    def draw(shape):
        return raw(rng.standard_normal(shape).astype(np.float32), dtype)
    q, key, val = draw((T, hq, d)), draw((T, hkv, d)), draw((T, hkv, d))
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[7] = -1
    pos = rng.integers(0, maxpos, size=T).astype(np.int32)
    cos, sin = W.rope_tables(maxpos, d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd = torch.from_numpy(q.view(np.int16) if dtype == "bf16" else q).to(DEV).view(tdt)
    kd = torch.from_numpy(key.view(np.int16) if dtype == "bf16" else key).to(DEV).view(tdt)
    vd = torch.from_numpy(val.view(np.int16) if dtype == "bf16" else val).to(DEV).view(tdt)
    kcd = torch.from_numpy(kp.view(np.int16) if dtype == "bf16" else kp).to(DEV).view(tdt)
    vcd = torch.from_numpy(vp.view(np.int16) if dtype == "bf16" else vp).to(DEV).view(tdt)
    qo = torch.empty_like(qd)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    say(f"[case] rope cache write {dtype} d{d}: T={T} hq={hq} hkv={hkv}")
    pa.pa_rope_reshape_and_cache(qo, qd, kd, vd, kcd, vcd, torch.from_numpy(slots).to(DEV),
                                 torch.from_numpy(pos).to(DEV), torch.from_numpy(cos).to(DEV),
                                 torch.from_numpy(sin).to(DEV), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    same = _rope.check(dtype, host_raw(qo), host_raw(kcd), host_raw(vcd), q, key, val, kp, vp, slots, pos, cos, sin)
    assert same > 0.99 or dtype == "f32"
    # in place on q gives the same bytes
    pa.pa_rope_reshape_and_cache(qd, qd, kd, vd, kcd, vcd, torch.from_numpy(slots).to(DEV),
                                 torch.from_numpy(pos).to(DEV), torch.from_numpy(cos).to(DEV),
                                 torch.from_numpy(sin).to(DEV), status)
    torch.cuda.synchronize()
    assert np.array_equal(host_raw(qd), host_raw(qo))


def test_rope_then_attention(pa):
    """A mixed batch whose new tokens go through the rotary cache write (q rotated, keys rotated
    into their pages) and then through pa_forward; the oracle rotates q and the new keys itself,
    rounds them to bfloat16 as the pool stores them, and computes attention in float64."""
    from oracle import attention as oattn
    from tests import _rope
    from tests._gpu import TOL
    w = W.random_ragged(31, "bf16", 16, 4, 128, [1, 200, 1, 37], [900, 1500, 3000, 37], with_slots=True)
    q, kc, vc, nk, nv = W.make_values(w, DEV)
    maxpos = 4096
    cos, sin = W.rope_tables(maxpos, 128)
    ql = np.diff(w.query_start_loc)
    pos = np.concatenate([np.arange(L - n, L) for n, L in zip(ql, w.context_lens)]).astype(np.int32)
    qh, kh, vh, nkh, nvh = (host_raw(t) for t in (q, kc, vc, nk, nv))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    qr = torch.empty_like(q)
    say(f"[case] rope + attention: q_lens {list(ql)}, contexts {list(w.context_lens)}")
    pa.pa_rope_reshape_and_cache(qr, q, nk, nv, kc, vc, torch.from_numpy(w.new_slots).to(DEV),
                                 torch.from_numpy(pos).to(DEV), torch.from_numpy(cos).to(DEV),
                                 torch.from_numpy(sin).to(DEV), status)
    run = Run(w)
    out = run.forward(qr, kc, vc)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(run.status.item()) == 0
    q_ref, k_ref, v_ref, _, _ = _rope.expected("bf16", qh, nkh, nvh, kh, vh, w.new_slots, pos, cos, sin)
    ref = oattn.paged_attention(q_ref, k_ref, v_ref, w.block_tables, w.context_lens, w.query_start_loc,
                                w.scale, "bf16")
    got = to_f64(out)
    a, r = TOL["bf16"]
    ratio = float((np.abs(got - ref) / (a + r * np.abs(ref))).max())
    say(f"  worst err/bound {ratio:.3f}")
    assert np.isfinite(got).all() and ratio <= 1.0


@pytest.mark.parametrize("case", range(len(SHARED_CASES)))
def test_shared_prefix_forward(pa, case):
    """Decode groups sharing prompt pages through pa_forward_shared: every row against the
    fp64 oracle (plain attention over each sequence's own table) and against pa_forward."""
    seed, hq, hkv, d, spec, bad = SHARED_CASES[case]
    w, groups = shared_prefix_batch(seed, hq, hkv, d, spec, bad_group=bad)
    say(f"[case] shared prefixes {spec} hq={hq} hkv={hkv} d={d} bad={bad}")
    check_tables_in_pool(w)
    q, kc, vc, _, _ = W.make_values(w, DEV)
    r = Run(w)
    ref_out = r.forward(q, kc, vc)
    torch.cuda.synchronize()
    r.check_status()
    nbytes = pa.pa_forward_shared_workspace_bytes(w.num_seqs, len(groups), w.num_tokens, w.max_q_len, hq, hkv, d,
                                                  w.max_context_len, pa.PA_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    pa.pa_forward_shared(out, q, kc, vc, r.tables, r.lens, r.qsl, torch.from_numpy(groups).to(DEV), w.max_q_len,
                         w.max_context_len, w.scale, ws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == (pa.PA_DEV_BAD_GROUP if bad else 0)
    rows, ref = oracle_rows(w, q, kc, vc, range(w.num_seqs))
    got = to_f64(out)
    assert np.isfinite(got).all()
    assert_close(got[rows], ref, "bf16", f"shared case {case}")
    # the same attention as pa_forward, up to the rounding of the split
    a, rr = 2e-3, 1e-2
    plain = to_f64(ref_out)
    assert (np.abs(got - plain) <= a + rr * np.abs(plain)).all()


def test_streaming_sequences_attention(pa):
    """Attention sinks + sliding window (k = 4, w = 100): tokens stream through the
    allocator's slots into the pool; a second sequence forks at token 120 and goes on
    by itself (its first overwrite of the shared pages copies them).  At checkpoints one
    decode row per sequence attends its cache, compared with the oracle over exactly the
    sink tokens and the last w tokens of that sequence (kept on the host, independent
    of where the pages put them)."""
    from oracle import attention as oattn
    from tests._gpu import TOL
    H, d, k, w, NB = 8, 128, 4, 100, 64
    ks, vs = W.cache_shapes(NB, H, d, "bf16")
    gen = torch.Generator(device=DEV).manual_seed(9)
    kc = W.fill_normal(torch.empty(ks, dtype=torch.bfloat16, device=DEV), gen)
    vc = W.fill_normal(torch.empty(vs, dtype=torch.bfloat16, device=DEV), gen)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    alloc = pa.Allocator(NB, 16)
    alloc.create_streaming(0, k, w, 0)
    hist = {0: []}                                   # per sequence: host bf16 bits of every token's (K, V)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    a, r = TOL["bf16"]
    worst = 0.0
    for t in range(320):
        if t == 120:
            alloc.fork(0, 1)
            hist[1] = list(hist[0])
        for sq in sorted(hist):
            slot, cow = alloc.append_slot(sq)
            if cow:
                pa.pa_copy_blocks(kc, vc, torch.tensor([cow], dtype=torch.int32, device=DEV), status)
            kn = W.fill_normal(torch.empty((1, H, d), dtype=torch.bfloat16, device=DEV), gen)
            vn = W.fill_normal(torch.empty((1, H, d), dtype=torch.bfloat16, device=DEV), gen)
            pa.pa_reshape_and_cache(kn, vn, kc, vc, torch.tensor([slot], dtype=torch.int64, device=DEV), status)
            hist[sq].append((host_raw(kn)[0], host_raw(vn)[0]))
        if t in (50, 103, 104, 121, 200, 319):
            for sq in sorted(hist):
                n = len(hist[sq])
                L = alloc.num_tokens(sq)
                assert L == min(n, k + w)
                tab = alloc.block_tables([sq], (k + w + 15) // 16)
                q = W.fill_normal(torch.empty((1, H, d), dtype=torch.bfloat16, device=DEV), gen)
                nbytes = pa.pa_forward_workspace_bytes(1, 1, 1, H, H, d, L, pa.PA_BF16)
                ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
                out = torch.empty_like(q)
                pa.pa_forward(out, q, kc, vc, torch.from_numpy(tab).to(DEV),
                              torch.tensor([L], dtype=torch.int32, device=DEV),
                              torch.tensor([0, 1], dtype=torch.int32, device=DEV), 1, L, scale, ws, status)
                torch.cuda.synchronize()
                assert int(status.item()) == 0
                kept = list(range(min(k, n))) + list(range(max(min(k, n), n - w), n))
                K = np.stack([hist[sq][i][0] for i in kept])
                V = np.stack([hist[sq][i][1] for i in kept])
                ref = oattn.attend_sequence(to_f64_bits(host_raw(q)), to_f64_bits(K), to_f64_bits(V), scale)
                got = to_f64(out)
                ratio = float((np.abs(got - ref) / (a + r * np.abs(ref))).max())
                worst = max(worst, ratio)
                assert np.isfinite(got).all() and ratio <= 1.0, (t, sq, ratio)
    say(f"[case] streaming sinks+window: worst err/bound {worst:.3f}")
    alloc.close()


def to_f64_bits(bits):
    from oracle import layout
    return layout.to_f64(bits, "bf16")


def read_probe_case(pif):
    """Pages, a page list with one id outside the pool, and the sink the documented
    thread assignment gives: wavefront w XORs piece l, l+64, l+128, l+192 of its
    pages pif*w .. pif*w+pif-1, pif*(w+W) .. into lane l."""
    rng = np.random.default_rng(11)
    npool, n, grid = 300, 257, 3
    words = rng.integers(0, 2**31 - 1, size=npool * 1024, dtype=np.int64).astype(np.int32)
    ids = rng.integers(0, npool, size=n).astype(np.int32)
    ids[5] = npool + 4
    pages = words.view(np.uint32).reshape(npool, 4, 64, 4)  # [page][k][lane][component]
    want = np.zeros(grid * 256, dtype=np.uint32)
    nwaves = grid * 4
    for i, pid in enumerate(ids):
        wave = (i // pif) % nwaves
        page = pid if pid < npool else 0
        want[wave * 64:(wave + 1) * 64] ^= np.bitwise_xor.reduce(
            pages[page].transpose(1, 0, 2).reshape(64, 16), axis=1)
    return words, ids, grid, want


@pytest.mark.parametrize("pif,mode", [(2, 0), (1, 0), (4, 1), (8, 0), (4, 2), (4, 3), (4, 10)])
def test_read_pages_probe(pif, mode):
    """The measurement library's page reader visits each listed page once, in the documented
    assignment, for every depth and kind of load."""
    import ctypes
    from paged_kv_cache_57_amd import build as _b
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.pa_probe_read_pages.restype = ctypes.c_int32
    lib.pa_probe_read_pages.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p]
    say(f"[case] page-read probe: {pif} pages in flight, mode {mode}")
    words, ids, grid, want = read_probe_case(pif)
    pool = torch.from_numpy(words).to(DEV)
    dids = torch.from_numpy(ids).to(DEV)
    sink = torch.full((grid * 256,), -1, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    st = lib.pa_probe_read_pages(pool.data_ptr(), pool.numel() * 4, dids.data_ptr(), dids.numel(), sink.data_ptr(),
                                 grid, pif, mode, status.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("waves", [4, 16])
def test_lds_read_probe(waves):
    """The LDS read probe folds exactly the documented pieces: thread t of workgroup b reads
    entries (((i * 8 + k) * 64 + 512 w + l) mod 4096) of the array {e, 3e, e ^ 5, 7}."""
    import ctypes
    from paged_kv_cache_57_amd import build as _b
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.pa_probe_lds_read.restype = ctypes.c_int32
    lib.pa_probe_lds_read.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    grid, iters = 3, 5
    say(f"[case] LDS read probe: {waves} wavefronts per workgroup")
    sink = torch.full((grid * 64 * waves,), -1, dtype=torch.int32, device=DEV)
    assert lib.pa_probe_lds_read(sink.data_ptr(), grid, waves, iters, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    t = np.arange(64 * waves)
    wv, lane = t // 64, t % 64
    want = np.zeros(64 * waves, dtype=np.uint32)
    for i in range(iters):
        for k in range(8):
            e = (((i * 8 + k) * 64 + wv * 512 + lane) & 4095).astype(np.uint32)
            want ^= e ^ (e * np.uint32(3)) ^ (e ^ np.uint32(5)) ^ np.uint32(7)
    got = sink.cpu().numpy().view(np.uint32).reshape(grid, -1)
    assert all(np.array_equal(got[b], want) for b in range(grid))
    assert lib.pa_probe_lds_read(sink.data_ptr(), grid, 5, iters, None) != 0  # only 4, 8 or 16 wavefronts


@pytest.mark.parametrize("shared", [False, True])
def test_decode_step_native(pa, shared):
    """pa_decode_step (allocator + one upload + copy + cache write + attention in one
    call) against the same step composed from the single entry points on a twin pool
    and allocator: outputs and pool bytes bit-identical every step (the same kernels
    on the same inputs); the last step's rows also against the oracle on a host copy
    of the pool.  4 prompts x 4 branches (copy-on-write of the shared partial page),
    40 steps, 8 heads of 128, with (shared=True) the prompts' full pages as
    shared-prefix groups."""
    from oracle import attention as oattn
    spec = W.parallel_sampling_spec(3, prompts=4, lo=100, hi=600, branches=4, steps=40, num_blocks=512,
                                    heads=8, head_dim=128)
    P, B, NB, H, d = len(spec.prompt_lens), spec.branches, spec.num_blocks, spec.heads, spec.head_dim
    say(f"[case] native decode step shared={shared}: prompts {list(spec.prompt_lens)} x {B}, NB={NB}")
    ks, vs = W.cache_shapes(NB, H, d, "bf16")
    gen = torch.Generator(device=DEV).manual_seed(5)
    kc_a = W.fill_normal(torch.empty(ks, dtype=torch.bfloat16, device=DEV), gen)
    vc_a = W.fill_normal(torch.empty(vs, dtype=torch.bfloat16, device=DEV), gen)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    allocs = [pa.Allocator(NB, 16, 0.0, spec.initial_free_order) for _ in range(2)]
    ids = [p * B + b for p in range(P) for b in range(B)]
    n = len(ids)
    for al in allocs:
        for p, L in enumerate(spec.prompt_lens):
            al.create(p * B, int(L))
    slots = np.concatenate([allocs[0].slots(p * B, 0, int(L)) for p, L in enumerate(spec.prompt_lens)])
    knew = W.fill_normal(torch.empty((len(slots), H, d), dtype=torch.bfloat16, device=DEV), gen)
    vnew = W.fill_normal(torch.empty((len(slots), H, d), dtype=torch.bfloat16, device=DEV), gen)
    pa.pa_reshape_and_cache(knew, vnew, kc_a, vc_a, torch.from_numpy(slots.astype(np.int64)).to(DEV), status)
    kc_b, vc_b = kc_a.clone(), vc_a.clone()
    for al in allocs:
        for p in range(P):
            for b in range(1, B):
                al.fork(p * B, p * B + b)
    mbps = (int(spec.prompt_lens.max()) + spec.steps + 15) // 16
    groups = None
    if shared:
        groups = torch.tensor([[p * B, B, 16 * (int(L) // 16)] for p, L in enumerate(spec.prompt_lens)],
                              dtype=torch.int32, device=DEV)
        nbytes = pa.pa_forward_shared_workspace_bytes(n, P, n, 1, H, H, d, 16 * mbps, pa.PA_BF16)
    else:
        nbytes = pa.pa_forward_workspace_bytes(n, n, 1, H, H, d, 16 * mbps, pa.PA_BF16)
    ws_a = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    sb = pa.pa_decode_step_staging_bytes(n, mbps)
    host = torch.empty(sb, dtype=torch.uint8).pin_memory()
    dev = torch.empty(sb, dtype=torch.uint8, device=DEV)
    qsl = torch.arange(n + 1, dtype=torch.int32, device=DEV)
    scale = 1.0 / np.sqrt(d)
    out_a = torch.empty((n, H, d), dtype=torch.bfloat16, device=DEV)
    out_b = torch.empty_like(out_a)
    copies = 0
    for step in range(spec.steps):
        q = W.fill_normal(torch.empty((n, H, d), dtype=torch.bfloat16, device=DEV), gen)
        kn = W.fill_normal(torch.empty((n, H, d), dtype=torch.bfloat16, device=DEV), gen)
        vn = W.fill_normal(torch.empty((n, H, d), dtype=torch.bfloat16, device=DEV), gen)
        # composed: the single entry points one by one
        sl, pairs = allocs[0].append_slots(ids)
        if len(pairs):
            pa.pa_copy_blocks(kc_a, vc_a, torch.from_numpy(pairs).to(DEV), status)
            copies += len(pairs)
        pa.pa_reshape_and_cache(kn, vn, kc_a, vc_a, torch.from_numpy(sl).to(DEV), status)
        lens = np.array([allocs[0].num_tokens(s) for s in ids], np.int32)
        L = int(lens.max())
        tab = torch.from_numpy(allocs[0].block_tables(ids, (L + 15) // 16)).to(DEV)
        dl = torch.from_numpy(lens).to(DEV)
        if shared:
            pa.pa_forward_shared(out_a, q, kc_a, vc_a, tab, dl, qsl, groups, 1, L, scale, ws_a, status)
        else:
            pa.pa_forward(out_a, q, kc_a, vc_a, tab, dl, qsl, 1, L, scale, ws_a, status)
        # native: one call
        pa.pa_decode_step(allocs[1], ids, out_b, q, kn, vn, kc_b, vc_b, scale, mbps, host, dev, ws_b,
                          groups=groups, dev_status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, step
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"outputs differ at step {step}"
    assert copies > 0
    assert torch.equal(kc_a.view(torch.int16), kc_b.view(torch.int16))
    assert torch.equal(vc_a.view(torch.int16), vc_b.view(torch.int16))
    kh, vh = host_raw(kc_b), host_raw(vc_b)
    lens = np.array([allocs[1].num_tokens(s) for s in ids], np.int32)
    tables = allocs[1].block_tables(ids, (int(lens.max()) + 15) // 16)
    ref = oattn.paged_attention(host_raw(q), kh, vh, tables, lens, np.arange(n + 1, dtype=np.int32),
                                float(np.float32(scale)), "bf16")
    assert_close(to_f64(out_b), ref, "bf16", "native decode step, last step")
    say(f"  {spec.steps} steps bit-identical to the composed calls; copy-on-write pairs {copies}")


def test_forward_replayed_from_a_hip_graph(pa):
    """A cache write + pa_forward captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed with new q, new K/V and eager work and synchronisations between replays:
    every replay's output equals the eager calls' on the same inputs bit for bit, and
    the oracle on the last one.  Nothing in the path allocates, copies from the host or
    clears memory with a memset node (the planner zeroes its counters in a kernel)."""
    w = W.random_ragged(41, "bf16", 16, 4, 128, [1, 1, 24, 1, 200], [700, 33, 1100, 3000, 2300], with_slots=True)
    say(f"[case] HIP graph replay: S={w.num_seqs} T={w.num_tokens} GQA 16/4, chunks of 24 and 200 rows")
    check_tables_in_pool(w)
    q, kc, vc, nk, nv = W.make_values(w, DEV)
    r = Run(w)
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # warm-up off the default stream, as capture expects
        r.write(nk, nv, kc, vc)
        r.forward(q, kc, vc, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.write(nk, nv, kc, vc)
        r.forward(q, kc, vc, out)
    gen = torch.Generator(device=DEV).manual_seed(3)
    for rep in range(4):
        W.fill_normal(q, gen)                  # eager work between the replays
        W.fill_normal(nk, gen)
        W.fill_normal(nv, gen)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        r.write(nk, nv, kc, vc)                # the same two calls, eagerly
        ref_out = r.forward(q, kc, vc)
        r.check_status()
        assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep} differs"
    rows, ref = oracle_rows(w, q, kc, vc, range(w.num_seqs))
    assert_close(to_f64(got.index_select(0, torch.from_numpy(rows).to(DEV))), ref, "bf16", "graph replay")
