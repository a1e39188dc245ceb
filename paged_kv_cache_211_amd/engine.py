"""A small paged KV cache manager built on libpkv: block pools on the device,
the library's host block allocator, and the C ABI's write / copy / decode
calls.  No arithmetic of the method happens here; it orders the calls.

"Day 6/90 of Inference Engineering" (PagedAttention notes): the manager hands
out blocks as tokens arrive, shares prefix blocks between prompts, and keeps
one block table per sequence.
"""

from __future__ import annotations

import numpy as np
import torch

from . import (BlockAllocator, empty_pools, paged_attention_decode, paged_attention_decode_prefix,
               paged_attention_decode_prefix_step, paged_attention_decode_queue,
               paged_attention_decode_step, paged_attention_prefix_plan,
               paged_attention_decode_step_streamk, paged_attention_decode_streamk,
               paged_attention_partition_offsets, paged_attention_streamk_workers,
               paged_attention_streamk_workspace_bytes, paged_attention_tile_offsets,
               paged_attention_workspace_bytes, paged_kv_copy_blocks, paged_kv_swap_blocks,
               paged_kv_swap_blocks_memcpy,
               paged_kv_write)


class PagedKVCache:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                 dtype: torch.dtype, device="cuda", free_order=None, k_scale=1.0, v_scale=1.0,
                 fill_byte: int | None = None):
        self.num_blocks, self.H, self.D, self.bs = num_blocks, num_kv_heads, head_dim, block_size
        self.dtype, self.device = dtype, torch.device(device)
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.alloc = BlockAllocator(num_blocks, block_size, free_order)
        self.key_cache, self.value_cache = empty_pools(num_blocks, num_kv_heads, head_dim,
                                                       block_size, dtype, device)
        if fill_byte is not None:
            self.key_cache.view(torch.uint8).fill_(fill_byte)
            self.value_cache.view(torch.uint8).fill_(fill_byte)
        self._ws = None
        self._stage = None

    # -- allocation and writes ------------------------------------------------
    def add_seq(self, seq: int):
        self.alloc.add_seq(seq)

    def fork(self, parent: int, child: int):
        self.alloc.fork(parent, child)

    def append_many(self, items, stream=None, write=True):
        """items: [(seq, key [n, H, D], value [n, H, D]), ...] (device tensors).

        Allocates every token on the host, applies the copy-on-write block
        copies, then scatters all rows with one write (skipped with
        write=False: a fused decode step stores them itself).  Returns the
        slot mapping (numpy int32) in item order.
        """
        slots, cows, keys, vals = [], [], [], []
        for seq, k, v in items:
            s, c = self.alloc.append(seq, int(k.shape[0]))
            slots.append(s)
            if len(c):
                cows.append(c)
            if k.shape[0]:
                keys.append(k)
                vals.append(v)
        if cows:
            pairs = torch.from_numpy(np.concatenate(cows).astype(np.int32)).to(self.device)
            paged_kv_copy_blocks(self.key_cache, self.value_cache, pairs, stream=stream)
        sl = np.concatenate(slots).astype(np.int32) if slots else np.zeros(0, np.int32)
        if keys and write:
            K = torch.cat(keys) if len(keys) > 1 else keys[0]
            V = torch.cat(vals) if len(vals) > 1 else vals[0]
            self.write(K.contiguous(), V.contiguous(), torch.from_numpy(sl).to(self.device), stream)
        return sl

    # -- swapping to host memory -----------------------------------------------
    def host_pool(self, num_host_blocks: int):
        """Pinned host pools of num_host_blocks blocks for swapped-out sequences."""
        self.host_key, self.host_value = empty_pools(num_host_blocks, self.H, self.D, self.bs,
                                                     self.dtype, "cpu", pin=True)
        self.alloc.set_host_pool(num_host_blocks)

    def _pairs(self, pairs, stream):
        """The pair list on the device, uploaded on the stream that reads it
        (so the caching allocator never hands its memory to another stream
        while the copy may still read it)."""
        p = torch.from_numpy(np.ascontiguousarray(np.asarray(pairs, dtype=np.int32)))
        if stream is None:
            return p.to(self.device)
        with torch.cuda.stream(stream):
            return p.to(self.device)

    def swap_out(self, seq: int, stream=None, staged: bool = True):
        """Move seq's blocks to host slots; its device blocks become free.
        With a stream of its own the copy overlaps work on other streams
        (a decode of the sequences that stay); the caller orders any later
        write into the freed blocks after it (an event).  staged=True (the
        default): the blocks are gathered into a device staging pool (one
        launch, HBM to HBM) and moved to the host slots by one asynchronous
        copy per run of consecutive slots (paged_kv_swap_blocks_memcpy), so
        a decode beside it keeps its speed; swaps that use the staging pool
        must run on one stream.  staged=False: one kernel moves the blocks
        straight to the host slots."""
        pairs = self.alloc.swap_out(seq)
        if pairs:
            if staged:
                p = np.asarray(pairs, dtype=np.int32).reshape(-1, 2)
                sk, sv = self._staging(len(p), stream)
                idx = np.arange(len(p), dtype=np.int32)
                paged_kv_swap_blocks(sk, sv, self.key_cache, self.value_cache,
                                     self._pairs(np.stack([p[:, 0], idx], 1), stream), stream=stream)
                paged_kv_swap_blocks_memcpy(self.host_key, self.host_value, sk, sv,
                                         np.stack([idx, p[:, 1]], 1), stream=stream)
            else:
                paged_kv_swap_blocks(self.host_key, self.host_value, self.key_cache,
                                     self.value_cache, self._pairs(pairs, stream), stream=stream)
        return pairs

    def swap_in(self, seq: int, stream=None, staged: bool = True):
        """Move seq back into free device blocks; with a stream of its own,
        the caller orders seq's next decode after the copy (an event).
        staged=True: asynchronous copies bring the host slots into the
        staging pool, one launch scatters them to the device blocks."""
        pairs = self.alloc.swap_in(seq)
        if pairs:
            if staged:
                p = np.asarray(pairs, dtype=np.int32).reshape(-1, 2)
                sk, sv = self._staging(len(p), stream)
                idx = np.arange(len(p), dtype=np.int32)
                paged_kv_swap_blocks_memcpy(sk, sv, self.host_key, self.host_value,
                                         np.stack([p[:, 0], idx], 1), stream=stream)
                paged_kv_swap_blocks(self.key_cache, self.value_cache, sk, sv,
                                     self._pairs(np.stack([idx, p[:, 1]], 1), stream), stream=stream)
            else:
                paged_kv_swap_blocks(self.key_cache, self.value_cache, self.host_key,
                                     self.host_value, self._pairs(pairs, stream), stream=stream)
        return pairs

    def _staging(self, n, stream):
        """Device staging pools of >= n blocks (grown on demand, reused), made
        on the stream that uses them."""
        if self._stage is None or self._stage[0].shape[0] < n:
            if stream is None:
                self._stage = empty_pools(n, self.H, self.D, self.bs, self.dtype, self.device)
            else:
                with torch.cuda.stream(stream):
                    self._stage = empty_pools(n, self.H, self.D, self.bs, self.dtype, self.device)
        return self._stage

    def write(self, key, value, slot_mapping, stream=None):
        paged_kv_write(key, value, self.key_cache, self.value_cache, slot_mapping,
                       k_scale=self.k_scale, v_scale=self.v_scale, stream=stream)

    # -- tables -----------------------------------------------------------------
    def seq_lens(self, seqs) -> np.ndarray:
        return np.array([self.alloc.seq_len(s) for s in seqs], dtype=np.int32)

    def block_tables(self, seqs, width: int | None = None):
        lens = self.seq_lens(seqs)
        w = width or max(1, int(-(-lens.max() // self.bs)) if len(lens) else 1)
        t = self.alloc.fill_tables(seqs, w, pad=-1)
        return torch.from_numpy(t).to(self.device)

    # -- decode -------------------------------------------------------------------
    def decode_inputs(self, seqs, partition_tokens: int = 0, streamk: bool = False,
                      num_q_heads: int | None = None, q_dtype=None, workers: int | None = None,
                      prefix: bool = False, prefix_min_blocks: int = 8):
        """Device tables, lengths and schedule metadata for a decode over seqs:
        split-K partitions of partition_tokens (0 = one pass), or with
        streamk=True the tile offsets and wave count of the stream-K schedule
        (num_q_heads and q_dtype needed; workers defaults to the resident
        waves of this device), or with prefix=True the shared-prefix plan for
        the runs of sequences whose tables share at least prefix_min_blocks
        leading blocks (partition_tokens > 0 and num_q_heads needed)."""
        lens = self.seq_lens(seqs)
        inp = {"block_tables": self.block_tables(seqs),
               "context_lens": torch.from_numpy(lens).to(self.device),
               "partition_tokens": int(partition_tokens), "partition_offsets": None,
               "total_partitions": 0, "lens_host": lens, "streamk": bool(streamk)}
        inp["prefix"] = None
        if prefix:
            go, gb = self.shared_prefix_groups(seqs, prefix_min_blocks)
            plan = paged_attention_prefix_plan(lens, go, gb, self.bs, partition_tokens,
                                               num_q_heads, self.H)
            inp["prefix"] = {k: torch.from_numpy(plan[k]).to(self.device)
                             for k in ("group_offsets", "group_prefix_blocks", "row_offsets",
                                       "suffix_offsets", "token_start", "prefix_item_offsets")}
            inp["prefix_totals"] = plan["totals"]
        if streamk:
            off, tot = paged_attention_tile_offsets(lens, self.bs)
            inp["tile_offsets"] = torch.from_numpy(off).to(self.device)
            inp["total_tiles"] = tot
            inp["workers"] = workers or paged_attention_streamk_workers(
                num_q_heads, self.H, self.D, self.bs, q_dtype, self.dtype)
        elif partition_tokens:
            off, tot = paged_attention_partition_offsets(lens, partition_tokens)
            inp["partition_offsets"] = torch.from_numpy(off).to(self.device)
            inp["total_partitions"] = tot
        return inp

    def shared_prefix_groups(self, seqs, min_blocks: int = 8):
        """Runs of consecutive sequences whose tables start with the same block
        ids (shared by reference, so identical contents): (group_offsets,
        group_prefix_blocks) for the shared-prefix decode.  A run is kept when
        it has at least two members and min_blocks shared blocks; every
        shared block is full (a shared, partly filled last block is copied on
        write before it is appended to)."""
        seqs = list(seqs)
        tabs = [self.alloc.block_table(s) for s in seqs]
        offs, blocks = [0], []
        i = 0
        while i < len(seqs):
            j, common = i + 1, len(tabs[i])
            while j < len(seqs):
                c = 0
                lim = min(common, len(tabs[j]))
                while c < lim and tabs[j][c] == tabs[i][c]:
                    c += 1
                if c < min_blocks:
                    break
                common = c
                j += 1
            if j - i < 2:
                common = 0
            # full blocks only: a member's last block may still be filling
            for k in range(i, j):
                common = min(common, (self.alloc.seq_len(seqs[k]) - 1) // self.bs if j - i > 1 else 0)
            offs.append(j)
            blocks.append(max(common, 0))
            i = j
        return np.array(offs, np.int32), np.array(blocks, np.int32)

    def _scratch(self, need):
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.device)
        return self._ws

    def workspace(self, total_partitions, num_q_heads, head_dim):
        """Device scratch for split-K partials (grown on demand, reused)."""
        return self._scratch(paged_attention_workspace_bytes(total_partitions, num_q_heads, head_dim))

    def streamk_workspace(self, inp, num_q_heads):
        S = len(inp["lens_host"])
        return self._scratch(paged_attention_streamk_workspace_bytes(inp["workers"], S, num_q_heads,
                                                                     self.H, self.D))

    def reserve_step(self, seqs, stream=None):
        """Allocate one new token for each sequence (copy-on-write included)
        without storing it; returns the slots.  decode_step stores the rows."""
        slots, cows = [], []
        for seq in seqs:
            sl, c = self.alloc.append(seq, 1)
            slots.append(sl)
            if len(c):
                cows.append(c)
        if cows:
            pairs = torch.from_numpy(np.concatenate(cows).astype(np.int32)).to(self.device)
            paged_kv_copy_blocks(self.key_cache, self.value_cache, pairs, stream=stream)
        return np.concatenate(slots).astype(np.int32) if slots else np.zeros(0, np.int32)

    def decode_step(self, query, new_key, new_value, inp, scale, out=None, stream=None):
        """Store row s of new_key/new_value as the last token of the s-th
        sequence of inp (already reserved), then decode; the store runs inside
        the decode launch where the kernel allows."""
        S, Hq, D = query.shape
        out = torch.empty_like(query) if out is None else out
        if inp.get("prefix") is not None:
            ws = self.workspace(inp["prefix_totals"][0], Hq, D)
            paged_attention_decode_prefix_step(out, query, new_key, new_value, self.key_cache,
                                               self.value_cache, inp["block_tables"],
                                               inp["context_lens"], scale, inp["partition_tokens"],
                                               inp["prefix"], inp["prefix_totals"], ws,
                                               k_scale=self.k_scale, v_scale=self.v_scale,
                                               stream=stream)
            return out
        if inp["streamk"]:
            paged_attention_decode_step_streamk(
                out, query, new_key, new_value, self.key_cache, self.value_cache,
                inp["block_tables"], inp["context_lens"], scale, inp["tile_offsets"],
                inp["total_tiles"], inp["workers"], self.streamk_workspace(inp, Hq),
                k_scale=self.k_scale, v_scale=self.v_scale, stream=stream)
            return out
        ws = None
        if inp["partition_tokens"]:
            ws = self.workspace(inp["total_partitions"], Hq, D)
        paged_attention_decode_step(out, query, new_key, new_value, self.key_cache,
                                    self.value_cache, inp["block_tables"], inp["context_lens"],
                                    scale, k_scale=self.k_scale, v_scale=self.v_scale,
                                    partition_tokens=inp["partition_tokens"],
                                    partition_offsets=inp["partition_offsets"],
                                    total_partitions=inp["total_partitions"], workspace=ws,
                                    stream=stream)
        return out

    def decode(self, query, inp, scale, out=None, stream=None, queue=False):
        """Decode with the schedule inp describes; queue=True takes split-K's
        work-counter form (paged_attention_decode_queue)."""
        S, Hq, D = query.shape
        out = torch.empty_like(query) if out is None else out
        if inp.get("prefix") is not None:
            ws = self.workspace(inp["prefix_totals"][0], Hq, D)
            paged_attention_decode_prefix(out, query, self.key_cache, self.value_cache,
                                          inp["block_tables"], inp["context_lens"], scale,
                                          inp["partition_tokens"], inp["prefix"],
                                          inp["prefix_totals"], ws, k_scale=self.k_scale,
                                          v_scale=self.v_scale, stream=stream)
            return out
        if inp["streamk"]:
            paged_attention_decode_streamk(out, query, self.key_cache, self.value_cache,
                                           inp["block_tables"], inp["context_lens"], scale,
                                           inp["tile_offsets"], inp["total_tiles"], inp["workers"],
                                           self.streamk_workspace(inp, Hq), k_scale=self.k_scale,
                                           v_scale=self.v_scale, stream=stream)
            return out
        ws = None
        if inp["partition_tokens"]:
            ws = self.workspace(inp["total_partitions"], Hq, D)
        fn = paged_attention_decode_queue if queue else paged_attention_decode
        fn(out, query, self.key_cache, self.value_cache, inp["block_tables"], inp["context_lens"],
           scale, k_scale=self.k_scale, v_scale=self.v_scale,
           partition_tokens=inp["partition_tokens"], partition_offsets=inp["partition_offsets"],
           total_partitions=inp["total_partitions"], workspace=ws, stream=stream)
        return out
