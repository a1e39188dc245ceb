"""Pins of the allocator specification model: the hand-traced example and the
invariants the pages state, on random operation sequences."""

import json
import os

import numpy as np
import pytest

from oracle.alloc_model import AllocError, AllocModel, ERR_INVALID, ERR_NO_BLOCKS, ERR_SEQ


def test_hand_traced_example(golden_dir):
    with open(os.path.join(golden_dir, "alloc_trace.json")) as f:
        g = json.load(f)
    m = AllocModel(g["num_blocks"], g["block_size"], g["free_order"])
    for st in g["steps"]:
        op = st["op"]
        if op == "add":
            m.add_seq(st["seq"])
        elif op == "fork":
            m.fork(st["parent"], st["child"])
        elif op == "free":
            m.free_seq(st["seq"])
        elif op == "append":
            if "error" in st:
                before = (m.free_list(), [m.refcount(b) for b in range(g["num_blocks"])],
                          {s: m.table(s) for s in m.tables})
                with pytest.raises(AllocError) as e:
                    m.append(st["seq"], st["n"])
                assert e.value.code == st["error"]
                after = (m.free_list(), [m.refcount(b) for b in range(g["num_blocks"])],
                         {s: m.table(s) for s in m.tables})
                assert before == after
            else:
                slots, cow = m.append(st["seq"], st["n"])
                assert slots == st["slots"] and [list(p) for p in cow] == st["cow"], st
    fin = g["final"]
    assert {str(s): m.table(s) for s in m.tables} == fin["tables"]
    assert {str(s): m.length(s) for s in m.tables} == fin["lens"]
    assert [m.refcount(b) for b in range(g["num_blocks"])] == fin["refcounts"]
    assert m.free_list() == fin["free"]


def check_invariants(m: AllocModel):
    bs = m.bs
    holders = [0] * m.num_blocks
    for s, tab in m.tables.items():
        L = m.length(s)
        # one block per started group of bs tokens: fill before allocate
        assert len(tab) == -(-L // bs)
        # only the last block may be partly filled: unused slots <= bs - 1
        assert len(tab) * bs - L <= bs - 1 if tab else L == 0
        assert len(set(tab)) == len(tab)
        for b in tab:
            holders[b] += 1
    # a refcount is exactly the number of tables holding the block
    assert holders == [m.refcount(b) for b in range(m.num_blocks)]
    # free blocks are exactly those nobody holds
    free = m.free_list()
    assert sorted(free) == [b for b in range(m.num_blocks) if holders[b] == 0]
    assert len(set(free)) == len(free)


def test_random_op_sequences_keep_invariants():
    rng = np.random.default_rng(11)
    for trial in range(200):
        nb = int(rng.integers(1, 24))
        bs = int(rng.choice([1, 2, 4, 16]))
        m = AllocModel(nb, bs, rng.permutation(nb))
        live, nxt = [], 0
        for _ in range(60):
            r = rng.random()
            try:
                if r < 0.2 or not live:
                    m.add_seq(nxt)
                    live.append(nxt)
                    nxt += 1
                elif r < 0.35:
                    p = int(rng.choice(live))
                    m.fork(p, nxt)
                    live.append(nxt)
                    nxt += 1
                elif r < 0.9:
                    s = int(rng.choice(live))
                    n = int(rng.integers(0, 3 * bs + 1))
                    need_free = m.num_free()
                    L0, tab0 = m.length(s), m.table(s)
                    slots, cows = m.append(s, n)
                    assert len(slots) == n and m.length(s) == L0 + n
                    assert len(cows) <= 1
                    # every slot lands in the sequence's own table at its position
                    tab = m.table(s)
                    for k, sl in enumerate(slots):
                        pos = L0 + k
                        assert sl == tab[pos // bs] * bs + pos % bs
                    # never write into a block somebody else still holds
                    for sl in slots:
                        assert m.refcount(sl // bs) == 1
                    # shared full blocks stay shared; only the partly-filled
                    # shared last block is copied
                    if cows:
                        assert L0 % bs != 0 and cows[0][0] == tab0[-1]
                else:
                    s = int(rng.choice(live))
                    m.free_seq(s)
                    live.remove(s)
            except AllocError as e:
                assert e.code == ERR_NO_BLOCKS
            check_invariants(m)


def test_allocation_succeeds_whenever_enough_blocks_are_free():
    # external fragmentation is gone: any free block serves any sequence
    rng = np.random.default_rng(12)
    for _ in range(50):
        nb, bs = 16, 4
        m = AllocModel(nb, bs, rng.permutation(nb))
        m.add_seq(0)
        m.append(0, int(rng.integers(0, nb * bs // 2)))
        m.add_seq(1)
        room = m.num_free() * bs
        m.append(1, room)           # exactly fills the pool
        assert m.num_free() == 0
        with pytest.raises(AllocError):
            m.append(1, 1)


def test_errors_leave_state_unchanged():
    m = AllocModel(4, 2, [3, 1, 0, 2])
    m.add_seq(5)
    m.append(5, 3)
    snap = (m.free_list(), m.table(5), m.length(5))
    with pytest.raises(AllocError) as e:
        m.append(5, 10)
    assert e.value.code == ERR_NO_BLOCKS
    assert (m.free_list(), m.table(5), m.length(5)) == snap
    for bad, code in [(lambda: m.append(9, 1), ERR_SEQ), (lambda: m.add_seq(5), ERR_SEQ),
                      (lambda: m.fork(9, 10), ERR_SEQ), (lambda: m.fork(5, 5), ERR_SEQ),
                      (lambda: m.free_seq(9), ERR_SEQ), (lambda: m.append(5, -1), ERR_INVALID)]:
        with pytest.raises(AllocError) as e:
            bad()
        assert e.value.code == code
    assert (m.free_list(), m.table(5), m.length(5)) == snap
    with pytest.raises(AllocError):
        AllocModel(3, 2, [0, 0, 1])


def test_full_shared_block_is_not_copied():
    m = AllocModel(6, 4, range(6))
    m.add_seq(0)
    m.append(0, 8)                  # two full blocks
    m.fork(0, 1)
    slots, cows = m.append(1, 1)    # next token opens a new block, no copy
    assert cows == [] and slots == [2 * 4]
    assert m.refcount(0) == 2 and m.refcount(1) == 2


def test_swap_hand_traced_example():
    """Traced by hand from the rules: FIFO device and host free lists,
    swap pairs in table order, LRU by the last add/fork/append/swap_in/touch."""
    m = AllocModel(4, 2, [2, 0, 3, 1])
    m.set_host_pool(3)
    m.add_seq(0)
    assert m.append(0, 3) == ([4, 5, 0], [])
    m.add_seq(1)
    assert m.append(1, 1) == ([6], [])
    assert m.lru() == 0
    assert m.swap_out(0) == [(2, 0), (0, 1)]
    assert m.free_list() == [1, 2, 0] and list(m.host_free) == [2]
    assert m.table(0) == [0, 1] and m.is_swapped(0) and m.length(0) == 3
    with pytest.raises(AllocError) as e:
        m.append(0, 1)                       # swapped out: invalid
    assert e.value.code == ERR_INVALID
    assert m.append(1, 2) == ([7, 2], [])
    with pytest.raises(AllocError) as e:
        m.swap_out(1)                        # 2 blocks, 1 host slot
    assert e.value.code == ERR_NO_BLOCKS
    assert m.table(1) == [3, 1] and list(m.host_free) == [2]
    assert m.swap_in(0) == [(0, 2), (1, 0)]
    assert m.table(0) == [2, 0] and m.free_list() == [] and list(m.host_free) == [2, 0, 1]
    assert m.lru() == 1
    m.touch(1)
    assert m.lru() == 0
    m.free_seq(0)
    assert m.free_list() == [2, 0] and m.table(1) == [3, 1]


def test_lfu_hand_traced_example():
    """Least frequently used, traced by hand: add, fork (the child),
    append, swap_in and touch each count one use; the fewest uses wins, the
    oldest stamp breaks ties; sequences holding shared blocks never qualify.
    The trace ends where the two policies name different sequences."""
    m = AllocModel(6, 2, range(6))
    m.add_seq(0); m.append(0, 2)             # uses 2, stamp 2
    m.add_seq(1); m.append(1, 2); m.append(1, 1)   # uses 3, stamp 5
    assert (m.lru(), m.lfu()) == (0, 0)
    m.touch(0)                               # uses 3, stamp 6: a tie on uses
    assert (m.lru(), m.lfu()) == (1, 1)
    m.touch(0)                               # uses 4, stamp 7
    assert (m.lru(), m.lfu()) == (1, 1)
    m.touch(1)                               # uses 4, stamp 8: a tie, 0 older
    assert (m.lru(), m.lfu()) == (0, 0)
    m.touch(1); m.touch(1)                   # uses 6, stamp 10
    m.add_seq(2); m.append(2, 1)             # uses 2, stamp 12
    assert (m.lru(), m.lfu()) == (0, 2)
    m.fork(2, 3)                             # 2 and 3 share a block: neither qualifies
    assert (m.lru(), m.lfu()) == (0, 0)
    m.free_seq(0)
    assert (m.lru(), m.lfu()) == (1, 1)


def test_swap_rules_on_random_ops():
    """Random ops with swaps: every device block is held by resident tables
    only, host slots by swapped tables only, lengths survive swaps, and the
    contents that the emitted pairs move come back to the same sequence."""
    rng = np.random.default_rng(31)
    for trial in range(80):
        nb, nh = int(rng.integers(2, 16)), int(rng.integers(0, 12))
        bs = int(rng.choice([1, 2, 4]))
        m = AllocModel(nb, bs, rng.permutation(nb))
        m.set_host_pool(nh)
        dev = [None] * nb                   # content label of each device block
        host = [None] * nh
        label = {}                          # (seq, logical block) -> label it must hold
        live, nxt, order = [], 0, []        # order: test's own recency list
        uses = {}                           # the test's own use counts
        for step in range(60):
            r = rng.random()
            try:
                if r < 0.15 or not live:
                    m.add_seq(nxt); live.append(nxt); order.append(nxt); uses[nxt] = 1; nxt += 1
                elif r < 0.25:
                    p = int(rng.choice(live))
                    m.fork(p, nxt)
                    for j in range(len(m.table(nxt))):
                        label[(nxt, j)] = label[(p, j)]
                    live.append(nxt); order.append(nxt); uses[nxt] = 1; nxt += 1
                elif r < 0.55:
                    s = int(rng.choice(live))
                    before = len(m.table(s)) if not m.is_swapped(s) else None
                    slots, cows = m.append(s, int(rng.integers(1, 3 * bs + 1)))
                    for src, dst in cows:
                        dev[dst] = dev[src]
                    for j, b in enumerate(m.table(s)):
                        if j >= before:
                            dev[b] = label[(s, j)] = (trial, step, s, j)
                    order.remove(s); order.append(s); uses[s] += 1
                elif r < 0.7:
                    s = int(rng.choice(live))
                    for b, h in m.swap_out(s):
                        host[h] = dev[b]
                elif r < 0.85:
                    s = int(rng.choice(live))
                    for h, b in m.swap_in(s):
                        dev[b] = host[h]
                    order.remove(s); order.append(s); uses[s] += 1
                elif r < 0.9:
                    s = int(rng.choice(live))
                    m.touch(s); order.remove(s); order.append(s); uses[s] += 1
                else:
                    s = int(rng.choice(live))
                    m.free_seq(s); live.remove(s); order.remove(s); del uses[s]
                    for k in [k for k in label if k[0] == s]:
                        del label[k]
            except AllocError:
                pass
            # invariants
            holders = [0] * nb
            hosts = []
            for s, tab in m.tables.items():
                assert len(tab) == -(-m.length(s) // bs)
                if m.is_swapped(s):
                    hosts += tab
                    for j, h in enumerate(tab):
                        assert host[h] == label[(s, j)]
                else:
                    for j, b in enumerate(tab):
                        holders[b] += 1
                        assert dev[b] == label[(s, j)]
            assert holders == [m.refcount(b) for b in range(nb)]
            assert sorted(m.free_list()) == [b for b in range(nb) if holders[b] == 0]
            assert sorted(hosts + list(m.host_free)) == list(range(nh))
            # LRU: the oldest eligible sequence in the test's own recency order
            elig = [s for s in order if not m.is_swapped(s) and m.table(s)
                    and all(m.refcount(b) == 1 for b in m.table(s))]
            if elig:
                assert m.lru() == elig[0]
                # LFU: fewest uses by the test's own count, recency breaking ties
                assert m.lfu() == min(elig, key=lambda s: (uses[s], order.index(s)))
            else:
                with pytest.raises(AllocError):
                    m.lru()
                with pytest.raises(AllocError):
                    m.lfu()
