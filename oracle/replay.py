"""Replay a workload's allocator operations and writes on the oracle side.

Given a workload description (its operations, its pool size and free order,
and a ``values(stream, start, n)`` callable for the rows each append writes),
this builds the oracle's own pools: the specification allocator decides every
slot and copy-on-write pair, copies are applied before the tokens that follow
them are written, and each append's rows are scattered with ``write_kv``.
Nothing here comes from the HIP library.
"""

from __future__ import annotations

import numpy as np

from .alloc_model import AllocModel
from .layout import copy_blocks, empty_pools, write_kv


class OracleState:
    def __init__(self, wl, fill=None, only_seqs=None):
        c = wl.cfg
        self.cfg = c
        self.model = AllocModel(wl.num_blocks, c.bs, wl.free_order)
        self.kc, self.vc = empty_pools(wl.num_blocks, c.H_kv, c.d, c.bs, c.kv_dtype, fill=fill)
        self.only = None if only_seqs is None else set(int(s) for s in only_seqs)
        self.cow_log = []

    def run(self, wl, ops):
        """Apply ops; returns the slot mapping of every append, in op order."""
        c = self.cfg
        slot_log = []
        for op in ops:
            kind = op[0]
            if kind == "add":
                self.model.add_seq(op[1])
            elif kind == "fork":
                self.model.fork(op[1], op[2])
            elif kind == "append":
                _, s, n, stream, start = op
                slots, cows = self.model.append(s, n)
                self.cow_log.extend(cows)
                copy_blocks(self.kc, self.vc, cows)
                slot_log.append(np.asarray(slots, dtype=np.int64))
                wanted = (self.only is None or stream[0] == "prefix" or s in self.only)
                if n and wanted:
                    k, v = wl.values(stream, start, n)
                    write_kv(self.kc, self.vc, k, v, slots, bs=c.bs, src_dtype=c.src_dtype,
                             cache_dtype=c.kv_dtype, k_scale=c.k_scale, v_scale=c.v_scale)
            else:
                raise ValueError(op)
        return slot_log

    def tables(self, S, width=None):
        """Block tables of sequences 0..S-1 padded with -1 to a common width."""
        rows = [self.model.table(s) for s in range(S)]
        w = width or max(1, max(len(r) for r in rows))
        out = np.full((S, w), -1, dtype=np.int64)
        for s, r in enumerate(rows):
            out[s, :len(r)] = r
        return out


def build(wl, fill=None, only_seqs=None):
    """Prefill and one decode step; returns (state, decode-step slot mapping)."""
    st = OracleState(wl, fill=fill, only_seqs=only_seqs)
    st.run(wl, wl.prefill)
    dec = st.run(wl, wl.decode)
    slot_mapping = np.concatenate(dec) if dec else np.zeros(0, dtype=np.int64)
    return st, slot_mapping
