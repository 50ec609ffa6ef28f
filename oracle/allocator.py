"""Ref-counted physical block allocator with per-sequence block tables (oracle side).

A Python mirror that the library's C++ allocator must match bit for bit
(block tables, slots, copy-on-write pairs, free counts, status codes).

Rules, with where they come from:

* Free list: a stack; allocation pops from its end, release pushes onto its
  end ("第7章：大模型部署实战" §2.3 BlockManager: ``free_blocks.pop()`` to
  allocate, ``free_blocks.append(...)`` to give a block back).  Its initial
  content is ``initial_free_order`` (default 0 .. N−1).
* ``create(seq, L)``: ⌈L/P⌉ blocks, allocated in logical order, each with
  reference count 1 ("大模型部署.md" §2.1 item 3 ``_allocate_sequence``;
  "第7章" §2.2.1 for ⌈L/P⌉).  All or nothing: without enough free blocks
  nothing changes.
* ``fork(parent, child)``: the child's table is a copy of the parent's and
  every shared block's count goes up by one (sharing of prompt blocks between
  samples of one prompt, "大模型部署.md" §2.1 item 4; the pages print no fork
  code — this is the plain reading).
* ``append_slot(seq)`` for the token that raises the length from L to L+1
  ("大模型部署.md" §2.1 item 3 ``append_slots``): if the table is one block
  short, take a fresh block; otherwise, if the last block is shared
  (count > 1), take a fresh block, put it in place of the last one, drop one
  reference from the old block and report the pair (old, new) for the
  device copy; otherwise nothing changes.  The new token's slot is
  ``table[L // P] · P + L % P``.
* ``free(seq)``: one reference less on each block in logical order; blocks
  reaching zero go back on the free stack in that order.
* ``can_allocate(n)``: with ``req = ⌈n/P⌉`` and watermark blocks
  ``wm = int(watermark · N)``: NEVER if ``N − req < wm``, OK if
  ``free − req ≥ wm``, else LATER ("大模型部署.md" §2.1 item 3 ``can_allocate``
  and ``watermark_blocks``).

Parity: pinned in tests by the pages' block_size=4 example ("第 15 章" §15.6:
a 4-token prompt fills one block, the fifth token opens a second, distinct
block), by ⌈L/P⌉ over a range of lengths, by the copy-on-write rule and by
ref-count invariants over random operation sequences.
"""
from __future__ import annotations

OK, LATER, NEVER = 0, 1, 2


class NoBlocks(RuntimeError):
    pass


class Allocator:
    def __init__(self, num_blocks: int, block_size: int = 16, watermark: float = 0.0,
                 initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0 or watermark < 0:
            raise ValueError("bad allocator arguments")
        self.N = num_blocks
        self.P = block_size
        self.wm = int(watermark * num_blocks)
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_free_order must be a permutation of 0..N-1")
        self.free = order
        self.ref = [0] * num_blocks
        self.tables = {}
        self.ntok = {}

    # -- queries
    def blocks_for(self, n_tokens: int) -> int:
        return (n_tokens + self.P - 1) // self.P

    def num_free(self) -> int:
        return len(self.free)

    def can_allocate(self, n_tokens: int) -> int:
        req = self.blocks_for(n_tokens)
        if self.N - req < self.wm:
            return NEVER
        if len(self.free) - req >= self.wm:
            return OK
        return LATER

    def block_table(self, seq):
        return list(self.tables[seq])

    def slots(self, seq, start: int, n: int):
        tab = self.tables[seq]
        if start < 0 or n < 0 or start + n > self.ntok[seq]:
            raise ValueError("slot range outside the sequence")
        return [tab[p // self.P] * self.P + p % self.P for p in range(start, start + n)]

    # -- mutations
    def _pop(self) -> int:
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def create(self, seq, n_tokens: int) -> None:
        if seq in self.tables:
            raise ValueError("sequence exists")
        if n_tokens < 0:
            raise ValueError("negative length")
        req = self.blocks_for(n_tokens)
        if req > len(self.free):
            raise NoBlocks("not enough free blocks")
        self.tables[seq] = [self._pop() for _ in range(req)]
        self.ntok[seq] = n_tokens

    def fork(self, parent, child) -> None:
        if parent not in self.tables:
            raise KeyError("unknown parent")
        if child in self.tables:
            raise ValueError("child exists")
        tab = list(self.tables[parent])
        for b in tab:
            self.ref[b] += 1
        self.tables[child] = tab
        self.ntok[child] = self.ntok[parent]

    def append_slot(self, seq):
        """Returns (slot, (old, new) or None) for the token at position ntok[seq]."""
        tab = self.tables[seq]
        L = self.ntok[seq]
        need = self.blocks_for(L + 1)
        cow = None
        if len(tab) < need:
            assert len(tab) == need - 1
            if not self.free:
                raise NoBlocks("no free block for the new token")
            tab.append(self._pop())
        elif self.ref[tab[-1]] > 1:
            if not self.free:
                raise NoBlocks("no free block for copy-on-write")
            old = tab[-1]
            new = self._pop()
            tab[-1] = new
            self.ref[old] -= 1
            cow = (old, new)
        self.ntok[seq] = L + 1
        return tab[L // self.P] * self.P + L % self.P, cow

    def free_seq(self, seq) -> None:
        tab = self.tables.pop(seq)
        del self.ntok[seq]
        for b in tab:
            if self.ref[b] <= 0:
                raise RuntimeError("reference count underflow")
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)


class PrefixCachingAllocator(Allocator):
    """The allocator with prefix caching ("大模型部署.md" §2.1 item 3,
    CachedBlockAllocator and LRUEvictor; "【自用】AI infra相关" part 二.4(2),
    prefix caching by block hashes).

    Rules, with where they come from and the readings taken:

    * Only full blocks are hashed.  The identity of full block j of a
      sequence is its whole token prefix (tokens 0 .. P(j+1)−1): the pages
      chain each block's hash with the previous block's, so two blocks match
      only when everything before them matches too.  The mirror uses that
      prefix itself as the key (no hash function, no collisions); the
      library uses a 64-bit chained hash and compares the block's own tokens
      and its parent's hash on a hit.
    * ``create_tokens(seq, tokens)``: every full block whose key is cached
      (in use by another sequence, or waiting in the evictor) is reused — one
      more reference, and a block in the evictor leaves it; every other
      block is new and a new full block is registered under its key.  Reused
      blocks are taken first, in logical order, then the new ones in logical
      order (reading: so that making room for a new block can never evict a
      block this same call reuses).  Returns the cached prefix length: P
      times the number of leading full blocks that were reused (the tokens
      the caller need not recompute; a non-aligned remainder is always
      recomputed, part 二.4(2)).  All or nothing.
    * A new block comes from the free stack; when that is empty, one block is
      evicted: in the evictor's insertion order, the first block, replaced by
      a later one with more hashed tokens while their access times are equal
      (LRUEvictor.evict).  Its key is forgotten.
    * ``free(seq)``: blocks whose count reaches zero go to the evictor when
      they carry a key (access time = the allocator's clock at that call;
      reading: the pages use the last access time, and a block is last used
      by the call that releases it) and to the free stack otherwise.
    * ``append_token(seq, token)``: as ``append_slot``; when the token fills
      the last block and the block's key is already cached by another block,
      the sequence switches to that block (one more reference; the filled
      block returns to the free stack, or, when it was shared, keeps its
      other users and no copy is made) — ``_maybe_promote_last_block``; when
      the key is not cached, the filled block (the copy, if it was shared) is
      registered under it.
    * ``num_free()`` counts free and evictor blocks (blocks in the evictor are
      available, part of the pages' account of usable blocks).
    * The clock advances by one at every mutating call.

    Sequences made by ``create`` (no tokens) never get keys; forks inherit
    their parent's tokens.
    """

    def __init__(self, num_blocks: int, block_size: int = 16, watermark: float = 0.0,
                 initial_free_order=None):
        super().__init__(num_blocks, block_size, watermark, initial_free_order)
        self.key = [None] * num_blocks          # block -> prefix key
        self.hashed_tokens = [0] * num_blocks   # tokens the key covers
        self.accessed = [0] * num_blocks
        self.cached = {}                        # key -> block
        self.evictor = []                       # blocks with a key and no reference, insertion order
        self.tokens = {}                        # seq -> token list (only sequences made with tokens)
        self.clock = 0

    # -- queries
    def num_free(self) -> int:
        return len(self.free) + len(self.evictor)

    def num_evictable(self) -> int:
        return len(self.evictor)

    def can_allocate(self, n_tokens: int) -> int:
        req = self.blocks_for(n_tokens)
        if self.N - req < self.wm:
            return NEVER
        if self.num_free() - req >= self.wm:
            return OK
        return LATER

    # -- helpers
    def _evict(self) -> int:
        cand = self.evictor[0]
        for b in self.evictor:
            if self.accessed[cand] < self.accessed[b]:
                break
            if self.hashed_tokens[cand] < self.hashed_tokens[b]:
                cand = b
        self.evictor.remove(cand)
        del self.cached[self.key[cand]]
        self.key[cand] = None
        self.hashed_tokens[cand] = 0
        return cand

    def _pop(self) -> int:
        b = self.free.pop() if self.free else self._evict()
        self.ref[b] = 1
        return b

    def _share(self, b: int) -> None:
        if self.ref[b] == 0:
            self.evictor.remove(b)
        self.ref[b] += 1

    def _register(self, b: int, key, ntok: int) -> None:
        self.key[b] = key
        self.hashed_tokens[b] = ntok
        self.cached[key] = b

    def _release(self, b: int) -> None:
        if self.ref[b] <= 0:
            raise RuntimeError("reference count underflow")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if self.key[b] is not None:
                self.accessed[b] = self.clock
                self.evictor.append(b)
            else:
                self.free.append(b)

    # -- mutations
    def create(self, seq, n_tokens: int) -> None:
        if seq in self.tables:
            raise ValueError("sequence exists")
        if n_tokens < 0:
            raise ValueError("negative length")
        req = self.blocks_for(n_tokens)
        if req > self.num_free():
            raise NoBlocks("not enough free blocks")
        self.clock += 1
        self.tables[seq] = [self._pop() for _ in range(req)]
        self.ntok[seq] = n_tokens

    def create_tokens(self, seq, tokens) -> int:
        tokens = [int(t) for t in tokens]
        if seq in self.tables:
            raise ValueError("sequence exists")
        L, P = len(tokens), self.P
        nblk = self.blocks_for(L)
        keys = [tuple(tokens[:P * (j + 1)]) for j in range(L // P)]
        hits = [j for j, k in enumerate(keys) if k in self.cached]
        revive = sum(1 for j in hits if self.ref[self.cached[keys[j]]] == 0)
        if nblk - len(hits) > self.num_free() - revive:
            raise NoBlocks("not enough free blocks")
        self.clock += 1
        tab = [None] * nblk
        for j in hits:
            b = self.cached[keys[j]]
            self._share(b)
            tab[j] = b
        for j in range(nblk):
            if tab[j] is None:
                tab[j] = self._pop()
                if j < len(keys):
                    self._register(tab[j], keys[j], P * (j + 1))
        self.tables[seq] = tab
        self.ntok[seq] = L
        self.tokens[seq] = tokens
        lead = 0
        while lead < len(keys) and lead in set(hits):
            lead += 1
        return lead * P

    def fork(self, parent, child) -> None:
        super().fork(parent, child)
        self.clock += 1
        if parent in self.tokens:
            self.tokens[child] = list(self.tokens[parent])

    def append_slot(self, seq):
        """As the base allocator's; new blocks may come from the evictor."""
        if seq in self.tokens:
            raise ValueError("a sequence made with tokens appends with append_token")
        tab = self.tables[seq]
        L = self.ntok[seq]
        need = self.blocks_for(L + 1)
        if (len(tab) < need or self.ref[tab[-1]] > 1) and self.num_free() == 0:
            raise NoBlocks("no free block")
        self.clock += 1
        cow = None
        if len(tab) < need:
            tab.append(self._pop())
        elif self.ref[tab[-1]] > 1:
            old = tab[-1]
            new = self._pop()
            tab[-1] = new
            self.ref[old] -= 1
            cow = (old, new)
        self.ntok[seq] = L + 1
        return tab[L // self.P] * self.P + L % self.P, cow

    def append_token(self, seq, token):
        """Returns (slot, (old, new) or None) for the token at position ntok[seq]."""
        if seq not in self.tables:
            raise KeyError("unknown sequence")
        if seq not in self.tokens:
            raise ValueError("append_token needs a sequence made with tokens")
        tab = self.tables[seq]
        L, P = self.ntok[seq], self.P
        toks = self.tokens[seq] + [int(token)]
        need = self.blocks_for(L + 1)
        fills = (L + 1) % P == 0
        key = tuple(toks) if fills else None
        hit = self.cached.get(key) if fills else None
        if len(tab) < need:
            if self.num_free() == 0:
                raise NoBlocks("no free block for the new token")
            self.clock += 1
            tab.append(self._pop())          # a new block holds one token: never full unless P == 1
            if fills:
                if hit is not None:
                    self._release(tab[-1])
                    self._share(hit)
                    tab[-1] = hit
                else:
                    self._register(tab[-1], key, L + 1)
            cow = None
        elif self.ref[tab[-1]] > 1:
            if hit is None and self.num_free() == 0:
                raise NoBlocks("no free block for copy-on-write")
            self.clock += 1
            old = tab[-1]
            if hit is not None:
                self._share(hit)
                self.ref[old] -= 1           # still held by another sequence
                tab[-1] = hit
                cow = None
            else:
                new = self._pop()
                self.ref[old] -= 1
                tab[-1] = new
                cow = (old, new)
                if fills:
                    self._register(new, key, L + 1)
        else:
            self.clock += 1
            if fills:
                if hit is not None:
                    self._share(hit)
                    self._release(tab[-1])
                    tab[-1] = hit
                else:
                    self._register(tab[-1], key, L + 1)
            cow = None
        self.ntok[seq] = L + 1
        self.tokens[seq] = toks
        return tab[L // P] * P + L % P, cow

    def free_seq(self, seq) -> None:
        if seq not in self.tables:
            raise KeyError("unknown sequence")
        tab = self.tables[seq]
        for b in tab:
            if self.ref[b] <= 0:
                raise RuntimeError("reference count underflow")
        self.clock += 1
        del self.tables[seq]
        del self.ntok[seq]
        self.tokens.pop(seq, None)
        for b in tab:
            self._release(b)


def streaming_append_position(seen: int, sinks: int, window: int) -> int:
    """Cache position of the token that raises a streaming sequence from `seen` to seen + 1
    tokens ("第 15 章：推理引擎与部署" §15.4, StreamingLLM: the first `sinks` tokens are
    kept, then only the most recent `window`).  The cache holds at most sinks + window
    tokens at positions 0 .. sinks + window - 1: the first sinks + window tokens take
    them in order; after that, token `seen` replaces the oldest window token, which sits
    at position sinks + (seen - sinks) mod window (a ring over the window positions).
    Attention is the same for any order of its keys, so the ring needs no reordering."""
    if seen < sinks + window:
        return seen
    return sinks + (seen - sinks) % window


class StreamingMixin:
    """Streaming sequences (sink tokens + sliding window) on the ref-counted allocator.

    * ``create_streaming(seq, sinks, window, n)``: n <= sinks + window tokens at
      positions 0 .. n-1, ⌈n/P⌉ blocks (the caller keeps a longer prompt's sinks
      and its last tokens).
    * ``append_streaming(seq)``: the new token's position is
      ``streaming_append_position``; while the cache grows, as ``append_slot``
      (a new block when the table is one short, copy-on-write of a shared last
      block); once full, the token overwrites a window position, and the block
      holding it is copied first when it is shared (copy-on-write of any block,
      not only the last).
    * ``num_tokens`` of a streaming sequence is the number of cached tokens,
      min(seen, sinks + window): the attention context length.
    """

    def _streaming_init(self):
        self.stream = {}   # seq -> [sinks, window, seen]

    def create_streaming(self, seq, sinks: int, window: int, n_tokens: int) -> None:
        if sinks < 0 or window <= 0 or n_tokens < 0 or n_tokens > sinks + window:
            raise ValueError("bad streaming parameters")
        self.create(seq, n_tokens)
        self.stream[seq] = [sinks, window, n_tokens]

    def append_streaming(self, seq):
        if seq not in self.tables:
            raise KeyError("unknown sequence")
        if seq not in self.stream:
            raise ValueError("not a streaming sequence")
        sinks, window, seen = self.stream[seq]
        cap = sinks + window
        if seen < cap:
            slot, cow = self.append_slot(seq)
        else:
            pos = streaming_append_position(seen, sinks, window)
            tab = self.tables[seq]
            j = pos // self.P
            cow = None
            if self.ref[tab[j]] > 1:
                if self.num_free() == 0:
                    raise NoBlocks("no free block for copy-on-write")
                old = tab[j]
                new = self._pop()
                self.ref[old] -= 1
                tab[j] = new
                cow = (old, new)
            slot = tab[j] * self.P + pos % self.P
        self.stream[seq][2] = seen + 1
        return slot, cow

    def fork(self, parent, child) -> None:
        super().fork(parent, child)
        if parent in self.stream:
            self.stream[child] = list(self.stream[parent])

    def free_seq(self, seq) -> None:
        super().free_seq(seq)
        self.stream.pop(seq, None)


class StreamingAllocator(StreamingMixin, Allocator):
    def __init__(self, *a, **k):
        super().__init__(*a, **k)
        self._streaming_init()
