"""Prefix caching end to end on the GPU ("大模型部署.md" §2.1 item 3, CachedBlockAllocator
and LRUEvictor; "【自用】AI infra相关" part 二.4(2): a later request reuses the cached
blocks of a matching prefix and only its uncached tokens are prefilled).

Requests are made from token ids on the library's allocator with prefix caching on.
A token's key and value rows are a function of its whole token prefix here, as they
are in a model (a seeded draw from a hash of tokens 0..p), so a reused page holds
exactly the rows the new request would have written.  Each request writes only the
tokens past its cached prefix, then attends them as a prefill chunk; decode steps go
through pa_decode_step with token ids, including steps where a filled page is
replaced by an equal cached one and steps that evict.  Every step: block tables,
slots and copy pairs against the prefix-caching mirror; every query row against the
fp64 oracle over a host copy of the pool; and the pool's pages against the rows the
prefixes define.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import allocator as mirror_alloc
from oracle import attention as oattn
from oracle import layout
from tests._gpu import DEV, assert_close, host_raw, say, to_f64
from tests._pools import bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_57_amd as pa
    assert torch.cuda.is_available()
    return pa

H, D, P = 8, 128, 16
MOD = (1 << 61) - 1


def prefix_hashes(tokens):
    """Rolling hash of every prefix tokens[0..p] (a seed for that token's K/V rows)."""
    out, h = [], 0
    for t in tokens:
        h = (h * 1000003 + int(t) + 1) % MOD
        out.append(h)
    return out


def kv_rows(tokens):
    """bf16 bits of the key and value rows [n, H, D] of each position of a token sequence."""
    ks, vs = [], []
    for h in prefix_hashes(tokens):
        x = np.random.default_rng(h).standard_normal((2, H, D)).astype(np.float32)
        ks.append(bf16_bits(x[0]))
        vs.append(bf16_bits(x[1]))
    return np.stack(ks), np.stack(vs)


def kv_last(tokens):
    """The rows of the last position only."""
    x = np.random.default_rng(prefix_hashes(tokens)[-1]).standard_normal((2, H, D)).astype(np.float32)
    return bf16_bits(x[0]), bf16_bits(x[1])


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


class State:
    def __init__(self, pa, nb, seed):
        self.pa = pa
        self.nb = nb
        self.rng = np.random.default_rng(seed)
        order = self.rng.permutation(nb).astype(np.int32)
        self.alloc = pa.Allocator(nb, P, 0.0, order)
        self.alloc.enable_prefix_caching()
        self.mirror = mirror_alloc.PrefixCachingAllocator(nb, P, 0.0, order)
        ks, vs = W.cache_shapes(nb, H, D, "bf16")
        g = torch.Generator(device=DEV).manual_seed(seed)
        self.kc = W.fill_normal(torch.empty(ks, dtype=torch.bfloat16, device=DEV), g)
        self.vc = W.fill_normal(torch.empty(vs, dtype=torch.bfloat16, device=DEV), g)
        self.status = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.tokens = {}
        self.scale = float(np.float32(1.0 / np.sqrt(D)))

    def check_tables(self, ids):
        for s in ids:
            assert self.alloc.block_table(s) == list(self.mirror.block_table(s)), s
            assert self.alloc.num_tokens(s) == self.mirror.ntok[s]
        assert self.alloc.num_free() == self.mirror.num_free()
        assert self.alloc.num_evictable() == self.mirror.num_evictable()

    def check_pages(self, ids):
        """Every position of every listed sequence holds the rows its prefix defines."""
        kh, vh = host_raw(self.kc), host_raw(self.vc)
        for s in ids:
            toks = self.tokens[s]
            K, V = kv_rows(toks)
            tab = self.alloc.block_table(s)
            for p in range(len(toks)):
                b, o = tab[p // P], p % P
                for h in range(H):
                    assert np.array_equal(layout.key_row(kh, b, h, o), K[p, h]), (s, p, h)
                    assert np.array_equal(layout.value_row(vh, b, h, o), V[p, h]), (s, p, h)

    def attend(self, ids, q_lens):
        """pa_forward over the listed sequences' last q_lens positions, against the oracle."""
        pa = self.pa
        lens = np.array([self.alloc.num_tokens(s) for s in ids], np.int32)
        qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        T = int(qsl[-1])
        cols = int((lens.max() + P - 1) // P)
        tables = self.alloc.block_tables(ids, cols)
        q = W.fill_normal(torch.empty((T, H, D), dtype=torch.bfloat16, device=DEV),
                          torch.Generator(device=DEV).manual_seed(int(self.rng.integers(1 << 30))))
        nbytes = pa.pa_forward_workspace_bytes(len(ids), T, int(max(q_lens)), H, H, D, int(lens.max()), pa.PA_BF16)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
        out = torch.empty_like(q)
        pa.pa_forward(out, q, self.kc, self.vc, torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV),
                      torch.from_numpy(qsl).to(DEV), int(max(q_lens)), int(lens.max()), self.scale, ws, self.status)
        torch.cuda.synchronize()
        assert int(self.status.item()) == 0
        ref = oattn.paged_attention(host_raw(q), host_raw(self.kc), host_raw(self.vc), tables, lens, qsl,
                                    self.scale, "bf16")
        return to_f64(out), ref

    def request(self, sid, tokens):
        """A new request: the allocator reuses what it can; only the uncached tokens are
        written, and they are attended as one prefill chunk."""
        cached = self.alloc.create_tokens(sid, tokens)
        assert cached == self.mirror.create_tokens(sid, tokens)
        self.tokens[sid] = list(tokens)
        n_new = len(tokens) - cached
        K, V = kv_rows(tokens)
        slots = self.alloc.slots(sid, cached, n_new)
        self.pa.pa_reshape_and_cache(dev_bf16(K[cached:]), dev_bf16(V[cached:]), self.kc, self.vc,
                                     torch.from_numpy(slots).to(DEV), self.status)
        got, ref = self.attend([sid], [n_new])
        assert_close(got, ref, "bf16", f"request {sid}: {len(tokens)} tokens, {cached} cached")
        return cached


def test_prefix_cached_requests_and_decode_steps(pa):
    st = State(pa, nb=56, seed=17)
    rng = st.rng
    A = [int(t) for t in rng.integers(0, 50000, size=200)]
    say("[case] prefix caching: requests sharing a prompt prefix, decode steps with token ids, eviction")
    assert st.request(0, A) == 0                                   # cold: every block new
    assert st.request(1, A[:160] + [int(t) for t in rng.integers(0, 50000, size=70)]) == 160
    assert st.request(2, A) == 192                                 # 12 full pages reused, 8 tokens written
    st.check_tables([0, 1, 2])
    st.check_pages([0, 1, 2])
    t0, t2 = st.alloc.block_table(0), st.alloc.block_table(2)
    assert t0[:12] == t2[:12] and t0[12] != t2[12]

    # decode steps through pa_decode_step with token ids: sequences 0 and 2 receive the
    # same tokens, so each page they fill has a cached twin and the later one switches to it
    ids = [0, 1, 2]
    mbps = 24
    sb = pa.pa_decode_step_staging_bytes(len(ids), mbps)
    host = torch.empty(sb, dtype=torch.uint8).pin_memory()
    dev = torch.empty(sb, dtype=torch.uint8, device=DEV)
    nbytes = pa.pa_forward_workspace_bytes(len(ids), len(ids), 1, H, H, D, P * mbps, pa.PA_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    switched = 0
    for step in range(56):
        tk = int(rng.integers(0, 3))
        new = [tk, int(rng.integers(0, 50000)), tk]
        before = [list(st.mirror.block_table(s)) for s in ids]
        for s, t in zip(ids, new):
            st.mirror.append_token(s, t)
            st.tokens[s].append(t)
        rows = [kv_last(st.tokens[s]) for s in ids]
        K = np.stack([kr for kr, _ in rows])
        V = np.stack([vr for _, vr in rows])
        q = W.fill_normal(torch.empty((len(ids), H, D), dtype=torch.bfloat16, device=DEV),
                          torch.Generator(device=DEV).manual_seed(100 + step))
        out = torch.empty_like(q)
        pa.pa_decode_step(st.alloc, ids, out, q, dev_bf16(K), dev_bf16(V), st.kc, st.vc, st.scale, mbps, host, dev,
                          ws, dev_status=st.status, token_ids=new)
        torch.cuda.synchronize()
        assert int(st.status.item()) == 0, step
        st.check_tables(ids)
        switched += sum(1 for i, s in enumerate(ids)
                        if len(before[i]) == len(st.mirror.block_table(s)) and before[i] != list(st.mirror.block_table(s)))
        lens = np.array([st.mirror.ntok[s] for s in ids], np.int32)
        tables = st.alloc.block_tables(ids, int((lens.max() + P - 1) // P))
        ref = oattn.paged_attention(host_raw(q), host_raw(st.kc), host_raw(st.vc), tables, lens,
                                    np.arange(len(ids) + 1, dtype=np.int32), st.scale, "bf16")
        got = to_f64(out)
        a, r = 2e-3, 1e-2
        assert np.isfinite(got).all() and (np.abs(got - ref) <= a + r * np.abs(ref)).all(), step
    assert switched > 0
    assert st.alloc.block_table(0)[:16] == st.alloc.block_table(2)[:16]
    st.check_pages(ids)
    say(f"  56 decode steps: tables equal the mirror's every step; {switched} filled pages switched to a cached twin")

    # release a request: its pages no other sequence holds wait in the evictor
    st.alloc.free(1)
    st.mirror.free_seq(1)
    st.tokens.pop(1)
    st.check_tables([0, 2])
    assert st.alloc.num_evictable() > 0
    # a long new prompt needs more pages than the free stack holds: the evictor gives some up
    free_stack = st.alloc.num_free() - st.alloc.num_evictable()
    n_new = P * (free_stack + 2) - 3
    C = [int(t) for t in rng.integers(0, 50000, size=n_new)]
    ev_before = st.alloc.num_evictable()
    assert st.request(3, C) == 0
    assert st.alloc.num_evictable() < ev_before
    st.check_tables([0, 2, 3])
    # request 1's prompt again: the pages still cached (shared with 0 and 2, or not evicted) come back
    again = A[:160] + [int(t) for t in rng.integers(0, 50000, size=37)]
    cached = st.request(4, again)
    assert cached >= 160
    st.check_tables([0, 2, 3, 4])
    st.check_pages([0, 2, 3, 4])
    say(f"  eviction: {ev_before - st.alloc.num_evictable()} pages evicted; a repeated prefix reused {cached} tokens")
    st.alloc.close()
