"""Parallel sampling with shared prompt pages, run against any backend and checked step by step.

Workflow ("大模型部署.md" §2.1 items 3-4: prompts share pages between samples,
a shared, partially filled last page is copied on write):

1. each prompt gets its pages from the allocator and its K/V are written
   through the allocator's slots;
2. every prompt is forked into ``branches`` sequences;
3. each decode step appends one token to every branch (allocator), copies
   the pages the allocator reports, writes the new K/V, and runs attention
   for one query row per branch.

An independent host pipeline (the oracle's allocator mirror and cache ops on
a host copy of the pool) runs alongside: slots, copy pairs and block tables
must be equal every step; at checkpoints the device pool bytes of every
referenced page must equal the host pool's, and the attention output must
match the oracle computed from the host pool.
"""
import numpy as np

from oracle import allocator as mirror_alloc
from oracle import attention as oattn
from oracle import cache_ops, layout

TOL = (2e-3, 1e-2)


def run_workflow(backend, spec, checkpoints, say=print):
    P, B, NB, H, d = len(spec.prompt_lens), spec.branches, spec.num_blocks, spec.heads, spec.head_dim
    alloc = backend.allocator(NB, spec.initial_free_order)
    mirror = mirror_alloc.Allocator(NB, 16, 0.0, spec.initial_free_order)
    kh, vh = backend.host_pools()                       # host copy of the starting pool bytes
    ids = [p * B + b for p in range(P) for b in range(B)]

    # 1. prompts
    for p, L in enumerate(spec.prompt_lens):
        alloc.create(p * B, int(L))
        mirror.create(p * B, int(L))
    slots = np.concatenate([alloc.slots(p * B, 0, int(L)) for p, L in enumerate(spec.prompt_lens)])
    want = np.concatenate([mirror.slots(p * B, 0, int(L)) for p, L in enumerate(spec.prompt_lens)])
    assert np.array_equal(slots, want)
    k_new, v_new = backend.randn((len(slots), H, d)), backend.randn((len(slots), H, d))
    backend.write(k_new, v_new, slots)
    cache_ops.reshape_and_cache(k_new.host, v_new.host, kh, vh, slots, inplace=True)

    # 2. forks
    for p in range(P):
        for b in range(1, B):
            alloc.fork(p * B, p * B + b)
            mirror.fork(p * B, p * B + b)

    worst = 0.0
    copies = 0
    for step in range(spec.steps):
        # 3a. one slot per branch, copy-on-write pairs
        slots, pairs = alloc.append_slots(ids)
        want_slots, want_pairs = [], []
        for s in ids:
            sl, cow = mirror.append_slot(s)
            want_slots.append(sl)
            if cow:
                want_pairs.append(cow)
        assert list(slots) == want_slots, step
        assert [tuple(x) for x in pairs] == want_pairs, step
        if len(pairs):
            backend.copy(pairs)
            cache_ops.copy_blocks(kh, vh, pairs, inplace=True)
            copies += len(pairs)
        # 3b. the new tokens' K/V
        k_new, v_new = backend.randn((len(ids), H, d)), backend.randn((len(ids), H, d))
        backend.write(k_new, v_new, np.asarray(slots))
        cache_ops.reshape_and_cache(k_new.host, v_new.host, kh, vh, np.asarray(slots), inplace=True)
        # 3c. tables every step, attention for one row per branch
        lens = np.array([mirror.ntok[s] for s in ids], np.int32)
        cap = int((lens.max() + 15) // 16)
        tables = alloc.block_tables(ids, cap)
        want_tab = np.full((len(ids), cap), -1, np.int32)
        for i, s in enumerate(ids):
            t = mirror.block_table(s)
            want_tab[i, :len(t)] = t
        assert np.array_equal(tables, want_tab), step
        q = backend.randn((len(ids), H, d))
        qsl = np.arange(len(ids) + 1, dtype=np.int32)
        out = backend.forward(q, tables, lens, qsl, int(lens.max()), 1.0 / np.sqrt(d))
        if step in checkpoints:
            used = sorted({int(b) for row in tables for b in row if b >= 0})
            kd, vd = backend.pages(used)
            assert np.array_equal(kd, kh[used]) and np.array_equal(vd, vh[used]), f"pool bytes differ at step {step}"
            ref = oattn.paged_attention(q.host, kh, vh, tables, lens, qsl,
                                        float(np.float32(1.0 / np.sqrt(d))), "bf16")
            got = layout.to_f64(backend.host(out), "bf16")
            ratio = float((np.abs(got - ref) / (TOL[0] + TOL[1] * np.abs(ref))).max())
            worst = max(worst, ratio)
            say(f"  step {step}: pages equal ({len(used)}), worst err/bound {ratio:.3f}")
            assert np.isfinite(got).all() and ratio <= 1.0, step
    return worst, copies


class Val:
    """A tensor value: backend handle plus the exact host bytes (bf16 bit patterns)."""

    def __init__(self, dev, host):
        self.dev = dev
        self.host = host


class GpuBackend:
    def __init__(self, pa, spec, seed=0):
        import torch

        import workloads as W
        from tests._gpu import DEV, host_raw
        self.pa, self.torch, self.W, self.DEV, self.host_raw = pa, torch, W, DEV, host_raw
        self.spec = spec
        ks, vs = W.cache_shapes(spec.num_blocks, spec.heads, spec.head_dim, "bf16")
        self.gen = torch.Generator(device=DEV).manual_seed(seed)
        self.kc = W.fill_normal(torch.empty(ks, dtype=torch.bfloat16, device=DEV), self.gen)
        self.vc = W.fill_normal(torch.empty(vs, dtype=torch.bfloat16, device=DEV), self.gen)
        self.status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def allocator(self, nb, order):
        return self.pa.Allocator(nb, 16, 0.0, order)

    def host_pools(self):
        return self.host_raw(self.kc).copy(), self.host_raw(self.vc).copy()

    def randn(self, shape):
        t = self.W.fill_normal(self.torch.empty(shape, dtype=self.torch.bfloat16, device=self.DEV), self.gen)
        return Val(t, self.host_raw(t))

    def write(self, k, v, slots):
        self.pa.pa_reshape_and_cache(k.dev, v.dev, self.kc, self.vc,
                                     self.torch.from_numpy(np.asarray(slots, np.int64)).to(self.DEV), self.status)

    def copy(self, pairs):
        self.pa.pa_copy_blocks(self.kc, self.vc,
                               self.torch.from_numpy(np.ascontiguousarray(pairs, np.int32)).to(self.DEV), self.status)

    def forward(self, q, tables, lens, qsl, max_ctx, scale):
        pa, torch, DEV = self.pa, self.torch, self.DEV
        S, T = len(lens), q.host.shape[0]
        nbytes = pa.pa_forward_workspace_bytes(S, T, 1, self.spec.heads, self.spec.heads, self.spec.head_dim,
                                               max_ctx, pa.PA_BF16)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
        out = torch.empty_like(q.dev)
        pa.pa_forward(out, q.dev, self.kc, self.vc, torch.from_numpy(tables).to(DEV),
                      torch.from_numpy(lens).to(DEV), torch.from_numpy(qsl).to(DEV), 1, max_ctx, scale, ws,
                      self.status)
        torch.cuda.synchronize()
        assert int(self.status.item()) == 0
        return out

    def pages(self, used):
        idx = self.torch.tensor(used, dtype=self.torch.int64, device=self.DEV)
        return self.host_raw(self.kc.index_select(0, idx)), self.host_raw(self.vc.index_select(0, idx))

    def host(self, out):
        return self.host_raw(out)


class EmuBackend:
    """Host pools driven through the CPU kernel emulator; allocator = libpa's C++ allocator."""

    def __init__(self, pa, spec, seed=0):
        from tests import _emu
        from tests._pools import empty_pools
        self.pa, self.emu, self.spec = pa, _emu, spec
        self.rng = np.random.default_rng(seed)
        self.kp, self.vp = empty_pools(self.rng, "bf16", spec.num_blocks, spec.heads, spec.head_dim)

    def allocator(self, nb, order):
        return self.pa.Allocator(nb, 16, 0.0, order)

    def host_pools(self):
        return self.kp.copy(), self.vp.copy()

    def randn(self, shape):
        from tests._pools import raw
        h = raw(self.rng.standard_normal(shape).astype(np.float32), "bf16")
        return Val(h, h)

    def write(self, k, v, slots):
        self.kp, self.vp, st = self.emu.reshape_and_cache("bf16", k.host, v.host, self.kp, self.vp, slots)
        assert st == 0

    def copy(self, pairs):
        self.kp, self.vp, st = self.emu.copy_blocks("bf16", self.kp, self.vp, pairs)
        assert st == 0

    def forward(self, q, tables, lens, qsl, max_ctx, scale):
        import workloads as W
        w = W.Workload("sampling", "bf16", self.spec.heads, self.spec.heads, self.spec.head_dim,
                       self.spec.num_blocks, lens, qsl, tables, float(np.float32(scale)))
        out, st = self.emu.forward(w, q.host, self.kp, self.vp)
        assert st == 0
        return out

    def pages(self, used):
        return self.kp[used], self.vp[used]

    def host(self, out):
        return out
