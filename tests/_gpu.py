"""Helpers for GPU parity tests: device inputs, host readback, oracle comparison."""
import os
import sys

import numpy as np
import torch

import workloads as W
from oracle import attention as oattn
from oracle import layout as olayout

DEV = torch.device("cuda:0")
# per-element bound |gpu - ref| <= ATOL + RTOL * |ref|
TOL = {"bf16": (2e-3, 1e-2), "f32": (1e-5, 1e-5)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host_raw(t):
    """Exact host copy of a device tensor: float32 as is, bfloat16 as uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dtype_name(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def to_f64(t):
    return olayout.to_f64(host_raw(t), dtype_name(t))


class Run:
    """Device copies of a workload's structure plus workspace and status word."""

    def __init__(self, w: W.Workload):
        self.w = w
        self.tables = torch.from_numpy(w.block_tables).to(DEV)
        self.lens = torch.from_numpy(w.context_lens).to(DEV)
        self.qsl = torch.from_numpy(w.query_start_loc).to(DEV)
        import paged_kv_cache_57_amd as pa
        code = pa.PA_BF16 if w.dtype == "bf16" else pa.PA_F32
        nbytes = pa.pa_forward_workspace_bytes(w.num_seqs, w.num_tokens, w.max_q_len, w.num_q_heads,
                                               w.num_kv_heads, w.head_dim, w.max_context_len, code)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
        self.status = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.slots = None if w.new_slots is None else torch.from_numpy(w.new_slots).to(DEV)

    def forward(self, q, k_cache, v_cache, out=None):
        import paged_kv_cache_57_amd as pa
        w = self.w
        if out is None:
            out = torch.empty_like(q)
        pa.pa_forward(out, q, k_cache, v_cache, self.tables, self.lens, self.qsl, w.max_q_len,
                      w.max_context_len, w.scale, self.workspace, self.status)
        return out

    def write(self, new_k, new_v, k_cache, v_cache):
        import paged_kv_cache_57_amd as pa
        pa.pa_reshape_and_cache(new_k, new_v, k_cache, v_cache, self.slots, self.status)

    def check_status(self):
        torch.cuda.synchronize()
        st = int(self.status.item())
        assert st == 0, f"device status flags {st:#x}"


def check_tables_in_pool(w: W.Workload):
    """Host-side precondition before launching: every referenced block lies in the pool."""
    for s, L in enumerate(w.context_lens):
        n = (int(L) + 15) // 16
        row = w.block_tables[s, :n]
        assert (row >= 0).all() and (row < w.num_blocks).all()
    assert w.block_tables.shape[1] * 16 >= w.max_context_len


def oracle_rows(w: W.Workload, q, k_cache, v_cache, seqs):
    """fp64 oracle output for all query rows of the listed sequences, reading only their blocks back."""
    seqs = list(seqs)
    lens = w.context_lens[seqs]
    need = sorted({int(b) for s, L in zip(seqs, lens) for b in w.block_tables[s, :(int(L) + 15) // 16]})
    idx = torch.tensor(need, dtype=torch.int64, device=DEV)
    kp = host_raw(k_cache.index_select(0, idx))
    vp = host_raw(v_cache.index_select(0, idx))
    remap = {b: i for i, b in enumerate(need)}
    mb = max(1, max((int(L) + 15) // 16 for L in lens))
    tabs = np.full((len(seqs), mb), -1, np.int32)
    for i, (s, L) in enumerate(zip(seqs, lens)):
        for j in range((int(L) + 15) // 16):
            tabs[i, j] = remap[int(w.block_tables[s, j])]
    qsl = w.query_start_loc
    rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs]).astype(np.int64)
    qlens = np.array([qsl[s + 1] - qsl[s] for s in seqs])
    sub_qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    qh = host_raw(q.index_select(0, torch.from_numpy(rows).to(DEV)))
    ref = oattn.paged_attention(qh, kp, vp, tabs, lens, sub_qsl, w.scale, w.dtype)
    return rows, ref


def assert_close(got_f64, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    err = np.abs(got_f64 - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    rel = err[np.abs(ref) >= 1e-3] / np.abs(ref[np.abs(ref) >= 1e-3])
    say(f"  {what}: max|err| {err.max():.3e}  max rel(|ref|>=1e-3) {rel.max() if rel.size else 0:.3e}  "
        f"bound {atol}+{rtol}|ref|  n={ref.size}")
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; worst at {i}: "
                             f"gpu {got_f64[i]!r} ref {ref[i]!r}")


def host_workers():
    """Threads for oracle work: the cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


_POOL = None


def oracle_pool():
    """The session's oracle worker processes (started on first use, shut down at exit)."""
    global _POOL
    if _POOL is None:
        import atexit
        from tests._oracle_pool import OraclePool
        _POOL = OraclePool(host_workers())
        atexit.register(_POOL.__exit__, None, None, None)
    return _POOL


def oracle_rows_all(w: W.Workload, q, k_cache, v_cache, seqs=None, batch_blocks=8000):
    """fp64 oracle output for every query row of the listed sequences (default: all),
    one oracle call per sequence, spread over worker processes.  Pages are read back
    in batches of at most batch_blocks blocks, so host memory stays bounded for pools
    of tens of GB.  Returns (rows, ref) like oracle_rows, rows in sequence order."""
    seqs = list(range(w.num_seqs)) if seqs is None else list(seqs)
    qsl = w.query_start_loc
    seqs = [s for s in seqs if qsl[s + 1] > qsl[s]]
    if not seqs:
        return np.zeros(0, np.int64), np.zeros((0, w.num_q_heads, w.head_dim))
    groups, cur, cur_n = [], [], 0
    for s in seqs:
        n = (int(w.context_lens[s]) + 15) // 16
        if cur and cur_n + n > batch_blocks:
            groups.append(cur)
            cur, cur_n = [], 0
        cur.append(s)
        cur_n += n
    groups.append(cur)
    rows_all, refs = [], []
    qh_all = host_raw(q)
    pool = oracle_pool()
    for grp in groups:
        need = np.unique(np.concatenate(
            [w.block_tables[s, :(int(w.context_lens[s]) + 15) // 16] for s in grp]).astype(np.int64))
        idx = torch.from_numpy(need).to(DEV)
        kp = host_raw(k_cache.index_select(0, idx))
        vp = host_raw(v_cache.index_select(0, idx))
        remap = np.full(w.num_blocks, -1, np.int64)
        remap[need] = np.arange(len(need))
        tasks = []
        for s in grp:
            L = int(w.context_lens[s])
            tab = remap[w.block_tables[s, :(L + 15) // 16].astype(np.int64)].astype(np.int32)
            a, b = int(qsl[s]), int(qsl[s + 1])
            tasks.append((qh_all[a:b], tab, L, w.scale, w.dtype))
        for s, ref in zip(grp, pool.run(kp, vp, tasks)):
            rows_all.append(np.arange(qsl[s], qsl[s + 1], dtype=np.int64))
            refs.append(ref)
        del kp, vp
    return np.concatenate(rows_all), np.concatenate(refs)
