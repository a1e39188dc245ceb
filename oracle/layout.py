"""Block-pool layout, slot scatter and block-table gather (oracle, test only).

The pages fix the idea, not a byte layout: the KV cache is cut into
fixed-size blocks placed anywhere in device memory, each sequence reaches its
blocks only through a block table, and each decode step writes the new token
into whatever block the manager handed out ("Day 6/90 of Inference
Engineering", PagedAttention notes; "PagedAttention Kernel：大模型推理优化的
显存管理革新" §1 and §2.1).  The element layout below is this project's
convention (the same one the HIP library uses, written here independently):

  key pool   : [num_blocks, H_kv, d // x, block_size, x]
  value pool : [num_blocks, H_kv, d, block_size]

with ``x = 16 // element_bytes`` (4 for fp32, 8 for bf16, 16 for fp8), so key
element (block b, head h, slot o, dim i) sits at ``[b, h, i // x, o, i % x]``
and value element at ``[b, h, i, o]``.  Token position t of a sequence lives
in block ``table[t // block_size]`` at slot ``t % block_size``; a slot id is
``block * block_size + slot``.

Pins (tests/test_oracle_layout.py): hand-written flat offsets for a small case
(tests/golden/layout_offsets.json); write-then-gather returns the written bits;
relabelling physical blocks by any permutation (moving the pool blocks with
them) leaves every gathered sequence unchanged; block copies and moves
between pools on pools whose blocks carry known byte patterns (listed
destinations take their sources' blocks whole, others keep theirs, a move
there and back restores the pool); the key scale routed to keys and the
value scale to values on an fp8 write, by hand-computed codes
(tests/test_oracle_fp8_scales.py).
"""

from __future__ import annotations

import numpy as np

from .formats import ELEM_BYTES, STORAGE, quantize_fp8


def pack_x(dtype: str) -> int:
    """Elements of one 16-byte key chunk."""
    return 16 // ELEM_BYTES[dtype]


def empty_pools(num_blocks: int, H_kv: int, d: int, bs: int, dtype: str, fill=None):
    """Allocate key and value pools in storage form; ``fill`` is a raw bit value."""
    x = pack_x(dtype)
    st = STORAGE[dtype]
    kc = np.zeros((num_blocks, H_kv, d // x, bs, x), dtype=st)
    vc = np.zeros((num_blocks, H_kv, d, bs), dtype=st)
    if fill is not None:
        if dtype == "f32":
            kc.view(np.uint32)[...] = fill
            vc.view(np.uint32)[...] = fill
        else:
            kc[...] = fill
            vc[...] = fill
    return kc, vc


def key_offset(b, h, o, i, *, H_kv, d, bs, dtype) -> int:
    """Flat element offset of key (b, h, o, i) in the key pool."""
    x = pack_x(dtype)
    return (((b * H_kv + h) * (d // x) + i // x) * bs + o) * x + i % x


def value_offset(b, h, o, i, *, H_kv, d, bs) -> int:
    """Flat element offset of value (b, h, o, i) in the value pool."""
    return ((b * H_kv + h) * d + i) * bs + o


def encode_for_cache(bits: np.ndarray, src_dtype: str, cache_dtype: str, scale: float) -> np.ndarray:
    """What a write stores: a bit copy, or fp8 quantise-on-write."""
    if cache_dtype == src_dtype:
        return np.asarray(bits, dtype=STORAGE[src_dtype])
    if cache_dtype == "fp8" and src_dtype in ("bf16", "f32"):
        return quantize_fp8(bits, src_dtype, scale)
    raise ValueError(f"unsupported write {src_dtype} -> {cache_dtype}")


def write_kv(kc, vc, key_bits, value_bits, slot_mapping, *, bs, src_dtype, cache_dtype,
             k_scale=1.0, v_scale=1.0):
    """Scatter token i's key/value rows ([T, H_kv, d]) into slot slot_mapping[i].

    A negative slot means "no token" and is skipped.  Every kv head of the
    token goes to the same (block, slot).
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots = slots[keep]
    if slots.size == 0:
        return
    kq = encode_for_cache(np.asarray(key_bits)[keep], src_dtype, cache_dtype, k_scale)
    vq = encode_for_cache(np.asarray(value_bits)[keep], src_dtype, cache_dtype, v_scale)
    x = pack_x(cache_dtype)
    T, H, d = kq.shape
    blk = slots // bs
    off = slots % bs
    # key: [b, h, i//x, o, i%x] <- k[t, h, i]
    kc[blk, :, :, off, :] = kq.reshape(T, H, d // x, x)
    # value: [b, h, i, o] <- v[t, h, i]
    vc[blk, :, :, off] = vq


def gather_seq(kc, vc, table_row, L: int, *, bs):
    """Keys and values of logical positions 0..L-1 through the block table.

    Returns raw stored bits shaped [L, H_kv, d] (token-major, like the
    contiguous cache a naive implementation would keep).
    """
    t = np.arange(L, dtype=np.int64)
    blk = np.asarray(table_row, dtype=np.int64)[t // bs]
    off = t % bs
    k = kc[blk, :, :, off, :]            # [L, H, d//x, x]
    v = vc[blk, :, :, off]               # [L, H, d]
    return k.reshape(L, k.shape[1], -1), v


def copy_blocks(kc, vc, pairs):
    """Copy whole key and value blocks src -> dst, in pair order."""
    for src, dst in pairs:
        kc[dst] = kc[src]
        vc[dst] = vc[src]


def move_blocks(dst_kc, dst_vc, src_kc, src_vc, pairs):
    """Copy whole key and value blocks between two pools of the same layout
    (a device pool and a host pool): dst[d] = src[s] for each pair (s, d)."""
    for src, dst in pairs:
        dst_kc[dst] = src_kc[src]
        dst_vc[dst] = src_vc[src]
