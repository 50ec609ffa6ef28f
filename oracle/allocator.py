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
