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

Swapping to host memory ("PagedAttention Kernel：大模型推理优化的显存管理革新"
§4.1 compares page replacement policies, but its table of them is missing
from the page, so the policy here is a reading, parity unpinned as a choice
of policy; only its stated rules below are pinned):
  * a host pool of ``num_host_blocks`` slots with its own FIFO free list
    (initially 0, 1, ..., popped from the front, returned to the back);
  * ``swap_out(seq)``: every block of the sequence must be unshared
    (refcount 1; shared blocks stay resident); table entry by entry, pop a
    host slot, record the pair (device block, host slot), drop the device
    block's reference (it returns to the device free list) and put the host
    slot in the table; the sequence is then swapped out;
  * ``swap_in(seq)``: table entry by entry, pop a device block, record the
    pair (host slot, device block), return the host slot to the host free
    list and put the device block in the table;
  * a swapped-out sequence can only be swapped in or freed (freeing returns
    its host slots in table order); other calls on it are invalid;
  * least recently used: a logical clock ticks on add, fork (the child),
    append, swap_in and touch, stamping that sequence; ``lru()`` names the
    resident sequence with at least one block, all of them unshared, whose
    stamp is oldest;
  * least frequently used ("PagedAttention Kernel…" §4.1 advises it for
    batch work, LRU for document processing): the same events count each
    sequence's uses, a new or forked sequence starting at one; ``lfu()``
    names, among the same candidates, the one with the fewest uses, the
    oldest stamp breaking ties.

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
        self.host_free: deque = deque()
        self.num_host = 0
        self.swapped: set[int] = set()
        self.stamp: dict[int, int] = {}
        self.uses: dict[int, int] = {}
        self.clock = 0

    # -- helpers ---------------------------------------------------------
    def _state(self):
        return (copy.copy(self.free), list(self.ref),
                {k: list(v) for k, v in self.tables.items()}, dict(self.lens))

    def _restore(self, st):
        self.free, self.ref, self.tables, self.lens = st

    def _tick(self, seq: int):
        self.clock += 1
        self.stamp[seq] = self.clock
        self.uses[seq] = self.uses.get(seq, 0) + 1

    def _resident(self, seq: int):
        if seq not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown sequence {seq}")
        if seq in self.swapped:
            raise AllocError(ERR_INVALID, f"sequence {seq} is swapped out")

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
        self._tick(seq)

    def fork(self, parent: int, child: int):
        if parent not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown parent {parent}")
        if child in self.tables:
            raise AllocError(ERR_SEQ, f"sequence {child} exists")
        self._resident(parent)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        self._tick(child)

    def append(self, seq: int, n: int):
        """Append n tokens; returns (slots [n], cow pairs [(src, dst), ...])."""
        self._resident(seq)
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
        self._tick(seq)
        return slots, cows

    def free_seq(self, seq: int):
        if seq not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown sequence {seq}")
        tab = self.tables.pop(seq)
        if seq in self.swapped:
            self.swapped.discard(seq)
            self.host_free.extend(tab)
        else:
            for b in tab:
                self._drop(b)
        del self.lens[seq]
        del self.stamp[seq]
        del self.uses[seq]

    def set_host_pool(self, num_host_blocks: int):
        if num_host_blocks < 0:
            raise AllocError(ERR_INVALID, "negative host pool size")
        if self.swapped:
            raise AllocError(ERR_INVALID, "sequences are swapped out")
        self.num_host = num_host_blocks
        self.host_free = deque(range(num_host_blocks))

    def swap_out(self, seq: int):
        """Move seq's blocks to host slots; returns [(device block, host slot), ...]."""
        self._resident(seq)
        tab = self.tables[seq]
        if any(self.ref[b] != 1 for b in tab):
            raise AllocError(ERR_INVALID, f"sequence {seq} holds shared blocks")
        if len(tab) > len(self.host_free):
            raise AllocError(ERR_NO_BLOCKS, "not enough free host slots")
        pairs = []
        for i, b in enumerate(tab):
            h = self.host_free.popleft()
            pairs.append((b, h))
            self._drop(b)
            tab[i] = h
        self.swapped.add(seq)
        return pairs

    def swap_in(self, seq: int):
        """Bring seq's blocks back; returns [(host slot, device block), ...]."""
        if seq not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown sequence {seq}")
        if seq not in self.swapped:
            raise AllocError(ERR_INVALID, f"sequence {seq} is resident")
        tab = self.tables[seq]
        if len(tab) > len(self.free):
            raise AllocError(ERR_NO_BLOCKS, "not enough free device blocks")
        pairs = []
        for i, h in enumerate(tab):
            b = self._pop()
            pairs.append((h, b))
            self.host_free.append(h)
            tab[i] = b
        self.swapped.discard(seq)
        self._tick(seq)
        return pairs

    def touch(self, seq: int):
        if seq not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown sequence {seq}")
        self._tick(seq)

    def _victims(self) -> list[int]:
        cands = [s for s, t in self.tables.items()
                 if s not in self.swapped and t and all(self.ref[b] == 1 for b in t)]
        if not cands:
            raise AllocError(ERR_SEQ, "no sequence can be swapped out")
        return cands

    def lru(self) -> int:
        return min(self._victims(), key=lambda s: self.stamp[s])

    def lfu(self) -> int:
        return min(self._victims(), key=lambda s: (self.uses[s], self.stamp[s]))

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

    def num_host_free(self) -> int:
        return len(self.host_free)

    def is_swapped(self, seq: int) -> bool:
        if seq not in self.tables:
            raise AllocError(ERR_SEQ, f"unknown sequence {seq}")
        return seq in self.swapped

    def free_list(self) -> list[int]:
        return list(self.free)
