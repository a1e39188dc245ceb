"""Specification model of the KV block allocator (oracle, test only).

What the pages fix ("Day 6/90 of Inference Engineering", PagedAttention
notes):
  * the cache manager hands out one block at a time during decode, and only
    when the tokens overflow the current block does a new block take the
    rest -- every block is filled before another is allocated, so deciding
    to allocate is just asking whether the last block is full;
  * nothing is reserved up front for a maximum length;
  * prompts with a common prefix share its blocks, and writing continues in
    a new block from the point where they differ;
  * a per-sequence block table maps logical blocks to scattered physical
    blocks.

What this model adds, as the plainest reading that makes tables unique (the
pages are silent on it):
  * the free list is a FIFO queue initialised from ``free_order``;
    allocation pops the front, a block whose refcount drops to 0 is pushed
    to the back;
  * ``fork`` copies the parent's table and length and adds one reference to
    every block in it;
  * ``append`` walks the new tokens one at a time: if the sequence has no
    block or its last block is full, pop a new block; otherwise, if the last
    block is shared (refcount > 1), pop a new block, record a copy-on-write
    pair (old, new), drop one reference to the old block and put the new
    block in its place; then the token takes slot
    ``table[pos // bs] * bs + pos % bs``;
  * ``free_seq`` drops one reference per table entry, in table order;
  * a call that fails leaves the state exactly as it was.

Pins (tests/test_oracle_alloc.py): the invariants the pages state (only the
last block of a sequence may be partly filled; block count = ceil(len/bs);
at most bs-1 unused slots per sequence; a refcount equals the number of
tables holding the block; allocation succeeds whenever enough blocks are
free, whatever their order) on random op sequences, and the hand-traced
prefix-sharing example in tests/golden/alloc_trace.json.
"""

from __future__ import annotations

import copy
from collections import deque

ERR_INVALID = -1
ERR_NO_BLOCKS = -5
ERR_SEQ = -6


class AllocError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


class AllocModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError(ERR_INVALID, "num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError(ERR_INVALID, "free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.bs = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}

    # -- helpers ---------------------------------------------------------
    def _state(self):
        return (copy.copy(self.free), list(self.ref),
                {k: list(v) for k, v in self.tables.items()}, dict(self.lens))

    def _restore(self, st):
        self.free, self.ref, self.tables, self.lens = st

    def _pop(self) -> int:
        if not self.free:
            raise AllocError(ERR_NO_BLOCKS, "no free blocks")
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def _drop(self, b: int):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    # -- operations ------------------------------------------------------
    def add_seq(self, seq: int):
        if seq in self.tables:
            raise AllocError(ERR_SEQ, f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0

    def fork(self, parent: int, child: int):
        if parent not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown parent {parent}")
        if child in self.tables:
            raise AllocError(ERR_SEQ, f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append(self, seq: int, n: int):
        """Append n tokens; returns (slots [n], cow pairs [(src, dst), ...])."""
        if seq not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown sequence {seq}")
        if n < 0:
            raise AllocError(ERR_INVALID, "negative token count")
        st = self._state()
        slots, cows = [], []
        try:
            tab = self.tables[seq]
            for _ in range(n):
                pos = self.lens[seq]
                if not tab or pos % self.bs == 0:
                    tab.append(self._pop())
                elif self.ref[tab[-1]] > 1:
                    new = self._pop()
                    old = tab[-1]
                    cows.append((old, new))
                    self._drop(old)
                    tab[-1] = new
                slots.append(tab[pos // self.bs] * self.bs + pos % self.bs)
                self.lens[seq] = pos + 1
        except AllocError:
            self._restore(st)
            raise
        return slots, cows

    def free_seq(self, seq: int):
        if seq not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown sequence {seq}")
        for b in self.tables.pop(seq):
            self._drop(b)
        del self.lens[seq]

    # -- queries ---------------------------------------------------------
    def table(self, seq: int) -> list[int]:
        if seq not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown sequence {seq}")
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        if seq not in self.lens:
            raise AllocError(ERR_SEQ, f"unknown sequence {seq}")
        return self.lens[seq]

    def refcount(self, block: int) -> int:
        return self.ref[block]

    def num_free(self) -> int:
        return len(self.free)

    def free_list(self) -> list[int]:
        return list(self.free)
