"""Seeded synthetic inputs for paged-attention runs.

This module only *draws* inputs: sequence lengths, the random permutation of
the physical block pool, the block tables cut from it, query row offsets, the
slot of every newly written token, and normally distributed tensor values.
It performs none of the attention, cache-write or allocator arithmetic; both
the CPU oracle and the GPU path consume what it produces.

Recipe (shared by every workload):

* Structure comes from ``numpy.random.default_rng(seed)`` in a fixed draw
  order: lengths first, then the pool permutation.
* Tensor values are N(0, 1), drawn in float32 by a ``torch.Generator`` seeded
  with ``seed`` on the target device and, for bf16 workloads, rounded to
  bfloat16 (round to nearest even).  Draw order: q, K pool, V pool, new K,
  new V.
* Sequence ``s`` takes the next ``blocks(L_s)`` entries of the permuted pool,
  in sequence order; table entries past a sequence's last block are -1.

Cache tensors use the library's block layout: keys as
``[num_blocks, kv_heads, head_dim // X, 16, X]`` with ``X = 16 // itemsize``
and values as ``[num_blocks, kv_heads, head_dim, 16]``.  Every (block, head)
tile is one contiguous run of ``16 * head_dim`` elements.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BLOCK = 16

__all__ = [
    "BLOCK", "Workload", "tiny_decode", "llama7b_decode", "gqa70b_decode",
    "gqa70b_long_decode", "splitfuse_mixed", "parallel_sampling_spec",
    "random_ragged", "alloc_cache", "fill_normal", "make_values",
]


def _blocks(n_tokens: int) -> int:
    # number of 16-token pages needed to hold n_tokens (structure only)
    return (int(n_tokens) + BLOCK - 1) // BLOCK


@dataclasses.dataclass
class Workload:
    """One batch of paged-attention inputs (host-side structure only)."""

    name: str
    dtype: str                      # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    context_lens: np.ndarray        # int32 [S]  keys visible to each sequence (new tokens included)
    query_start_loc: np.ndarray     # int32 [S+1] row offsets of each sequence's query tokens
    block_tables: np.ndarray        # int32 [S, max_blocks] physical block of each logical block
    scale: float                    # the float32 softmax scale handed to the kernel
    new_slots: Optional[np.ndarray] = None   # int64 [T] slot of each query token's new K/V (None: no cache write)
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_q_len(self) -> int:
        q = np.diff(self.query_start_loc)
        return int(q.max()) if q.size else 0

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int32)


def _tables_from_perm(lens, perm, max_blocks=None):
    nb = [_blocks(L) for L in lens]
    mb = max(nb) if max_blocks is None else max_blocks
    mb = max(mb, 1)
    tab = np.full((len(lens), mb), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(nb):
        tab[s, :n] = perm[off:off + n]
        off += n
    if off > len(perm):
        raise ValueError("pool too small for the requested lengths")
    return tab


def _scale(d):
    return float(np.float32(1.0 / np.sqrt(np.float32(d))))


def _new_slots(tables, lens, qlens):
    """Slot of each query token's new K/V: the last q_len positions of its sequence."""
    out = []
    for s, (L, q) in enumerate(zip(lens, qlens)):
        for pos in range(L - q, L):
            out.append(int(tables[s, pos // BLOCK]) * BLOCK + pos % BLOCK)
    return np.asarray(out, dtype=np.int64)


def tiny_decode(seed: int = 0) -> Workload:
    """Two fp32 sequences (37 and 100 keys), 4 MHA heads of dim 64, 32-block pool."""
    rng = np.random.default_rng(seed)
    lens = np.array([37, 100], dtype=np.int32)
    perm = rng.permutation(32).astype(np.int32)
    return Workload("tiny_decode_fp32", "f32", 4, 4, 64, 32, lens,
                    np.arange(3, dtype=np.int32), _tables_from_perm(lens, perm),
                    0.125, None, seed)


def llama7b_decode(seed: int = 0, batch: int = 64, lo: int = 512, hi: int = 4096,
                   num_blocks: int = 16384) -> Workload:
    """Batch-64 decode, 32 MHA heads of dim 128, bf16, lengths uniform in [512, 4096]."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    perm = rng.permutation(num_blocks).astype(np.int32)
    return Workload("llama7b_decode_b64", "bf16", 32, 32, 128, num_blocks, lens,
                    np.arange(batch + 1, dtype=np.int32), _tables_from_perm(lens, perm),
                    _scale(128), None, seed)


def gqa70b_decode(seed: int = 0, batch: int = 32, length: int = 2048,
                  num_blocks: int = 8192) -> Workload:
    """Batch-32 decode at 2048 keys, 64 query heads over 8 KV heads of dim 128, bf16."""
    rng = np.random.default_rng(seed)
    lens = np.full(batch, length, dtype=np.int32)
    perm = rng.permutation(num_blocks).astype(np.int32)
    return Workload("gqa70b_decode_b32_l2048", "bf16", 64, 8, 128, num_blocks, lens,
                    np.arange(batch + 1, dtype=np.int32), _tables_from_perm(lens, perm),
                    _scale(128), None, seed)


def gqa70b_long_decode(seed: int = 0, length: int = 32768, num_blocks: int = 4096) -> Workload:
    """One sequence of 32,768 keys, 64 query heads over 8 KV heads of dim 128, bf16."""
    rng = np.random.default_rng(seed)
    lens = np.array([length], dtype=np.int32)
    perm = rng.permutation(num_blocks).astype(np.int32)
    return Workload("gqa70b_decode_b1_l32768", "bf16", 64, 8, 128, num_blocks, lens,
                    np.arange(2, dtype=np.int32), _tables_from_perm(lens, perm),
                    _scale(128), None, seed)


def splitfuse_mixed(seed: int = 0, n_chunks: int = 2, chunk: int = 512, prior_hi: int = 8192,
                    n_decode: int = 1024, dec_lo: int = 128, dec_hi: int = 4096,
                    heads: int = 32, head_dim: int = 128, slack_blocks: int = 1024) -> Workload:
    """Dynamic-SplitFuse batch: prefill chunks continuing a cached prefix, then decodes.

    Chunk rows come first, then one row per decode sequence (query_start_loc
    order).  A chunk row at index i of a chunk with prior context c sits at
    position c + i.  Every query token also carries the slot its new K/V is
    written to, so the pass begins with a cache write of all T tokens.
    """
    rng = np.random.default_rng(seed)
    prior = rng.integers(0, prior_hi + 1, size=n_chunks)
    dec = rng.integers(dec_lo, dec_hi + 1, size=n_decode)
    lens = np.concatenate([prior + chunk, dec]).astype(np.int32)
    qlens = np.concatenate([np.full(n_chunks, chunk), np.ones(n_decode, dtype=np.int64)])
    nb = int(sum(_blocks(L) for L in lens)) + slack_blocks
    perm = rng.permutation(nb).astype(np.int32)
    tables = _tables_from_perm(lens, perm)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return Workload(f"splitfuse_{n_chunks}x{chunk}+{n_decode}dec", "bf16", heads, heads,
                    head_dim, nb, lens, qsl, tables, _scale(head_dim),
                    _new_slots(tables, lens, qlens), seed)


@dataclasses.dataclass
class ParallelSamplingSpec:
    """Structure of the shared-prefix parallel-sampling workflow."""

    prompt_lens: np.ndarray          # int32 [P]
    branches: int
    steps: int
    num_blocks: int
    initial_free_order: np.ndarray   # int32 [num_blocks]
    heads: int
    head_dim: int
    seed: int

    @property
    def scale(self) -> float:
        return _scale(self.head_dim)


def parallel_sampling_spec(seed: int = 0, prompts: int = 16, lo: int = 1000, hi: int = 4000,
                           branches: int = 4, steps: int = 256, num_blocks: int = 8192,
                           heads: int = 32, head_dim: int = 128) -> ParallelSamplingSpec:
    rng = np.random.default_rng(seed)
    plens = rng.integers(lo, hi + 1, size=prompts).astype(np.int32)
    order = rng.permutation(num_blocks).astype(np.int32)
    return ParallelSamplingSpec(plens, branches, steps, num_blocks, order, heads, head_dim, seed)


def random_ragged(seed: int, dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  q_lens, ctx_lens, slack_blocks: int = 8, with_slots: bool = False) -> Workload:
    """Arbitrary ragged batch (test shapes): explicit per-sequence query and context lengths."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(ctx_lens, dtype=np.int32)
    qlens = np.asarray(q_lens, dtype=np.int64)
    nb = int(sum(_blocks(L) for L in lens)) + slack_blocks
    perm = rng.permutation(nb).astype(np.int32)
    tables = _tables_from_perm(lens, perm)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    slots = _new_slots(tables, lens, qlens) if with_slots else None
    return Workload(f"ragged_s{seed}", dtype, num_q_heads, num_kv_heads, head_dim, nb, lens,
                    qsl, tables, _scale(head_dim), slots, seed)


# ---------------------------------------------------------------- tensor values

def _torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def cache_shapes(w_or_nb, kv_heads=None, head_dim=None, dtype=None):
    """Shapes of the key and value pools for the library's block layout."""
    if isinstance(w_or_nb, Workload):
        nb, kv_heads, head_dim, dtype = (w_or_nb.num_blocks, w_or_nb.num_kv_heads,
                                          w_or_nb.head_dim, w_or_nb.dtype)
    else:
        nb = w_or_nb
    x = 16 // (4 if dtype == "f32" else 2)
    return (nb, kv_heads, head_dim // x, BLOCK, x), (nb, kv_heads, head_dim, BLOCK)


def alloc_cache(w: Workload, device):
    import torch
    ks, vs = cache_shapes(w)
    td = _torch_dtype(w.dtype)
    return (torch.empty(ks, dtype=td, device=device), torch.empty(vs, dtype=td, device=device))


def fill_normal(t, gen, chunk_elems: int = 1 << 26):
    """Fill ``t`` in place with N(0,1) drawn in float32, rounded to t's dtype."""
    import torch
    flat = t.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e].copy_(torch.randn(e - s, generator=gen, dtype=torch.float32, device=t.device))
    return t


def make_values(w: Workload, device, fill_pool: bool = True):
    """Draw q, the K/V pools and (when the workload writes) the new K/V, in the fixed order."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    td = _torch_dtype(w.dtype)
    T = w.num_tokens
    q = fill_normal(torch.empty((T, w.num_q_heads, w.head_dim), dtype=td, device=device), gen)
    k_cache, v_cache = alloc_cache(w, device)
    if fill_pool:
        fill_normal(k_cache, gen)
        fill_normal(v_cache, gen)
    new_k = new_v = None
    if w.new_slots is not None:
        new_k = fill_normal(torch.empty((T, w.num_kv_heads, w.head_dim), dtype=td, device=device), gen)
        new_v = fill_normal(torch.empty((T, w.num_kv_heads, w.head_dim), dtype=td, device=device), gen)
    return q, k_cache, v_cache, new_k, new_v


def rope_tables(max_position: int, head_dim: int, base: float = 10000.0):
    """cos / sin tables [max_position][head_dim/2] in float32 for rotary embeddings:
    angle(p, i) = p · base^(-2i/head_dim), evaluated in float64 and rounded once."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
