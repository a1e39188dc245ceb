"""PagedAttention decode for AMD Instinct MI355X (gfx950).

Thin Python binding over libpkv.so (include/pkv.h): every function takes
torch tensors, checks that their shapes agree, and passes raw pointers, sizes
and the current HIP stream to the C ABI.  All computation happens in the
library's HIP kernels; nothing here computes attention, and there is no CPU
fallback.

    key_cache   [num_blocks, H_kv, head_dim // x, block_size, x]
    value_cache [num_blocks, H_kv, head_dim, block_size]
    x = 16 // element size (4 fp32, 8 bf16, 16 fp8)

fp8 pools are torch.uint8 (or torch.float8_e4m3fn) tensors of E4M3FN codes.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _native
from ._native import PKV_BF16, PKV_F32, PKV_FP8_E4M3, PkvError, check, lib

__all__ = [
    "PkvError", "paged_kv_write", "paged_attention_decode", "paged_attention_decode_partials",
    "paged_attention_decode_queue", "paged_kv_swap_blocks_memcpy",
    "paged_attention_splitk_reduce", "paged_kv_copy_blocks", "paged_kv_gather",
    "paged_attention_partition_offsets", "paged_attention_workspace_bytes", "BlockAllocator",
    "empty_pools", "cache_dtype_code", "pkv_hbm_read_probe", "pkv_paged_read_probe",
]

lib()  # fail at import if the library is missing or incomplete

_CODES = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16, torch.uint8: PKV_FP8_E4M3,
          torch.float8_e4m3fn: PKV_FP8_E4M3}


def cache_dtype_code(t: torch.Tensor) -> int:
    try:
        return _CODES[t.dtype]
    except KeyError:
        raise PkvError(-1, f"unsupported tensor dtype {t.dtype}") from None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise PkvError(-1, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise PkvError(-1, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PkvError(-1, f"{name} must be {dtype}, got {t.dtype}")


def _pool_shape(key_cache: torch.Tensor, value_cache: torch.Tensor):
    if key_cache.dim() != 5 or value_cache.dim() != 4:
        raise PkvError(-1, "key_cache must be 5-D and value_cache 4-D")
    nb, H, dx, bs, x = key_cache.shape
    D = dx * x
    if tuple(value_cache.shape) != (nb, H, D, bs) or value_cache.dtype != key_cache.dtype:
        raise PkvError(-1, f"value_cache shape {tuple(value_cache.shape)} does not match key_cache")
    if x * key_cache.element_size() != 16:
        raise PkvError(-1, "key_cache last dim must hold 16 bytes")
    return nb, H, D, bs


def empty_pools(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                dtype: torch.dtype, device="cuda", pin: bool = False):
    """Allocate (uninitialised) key and value pools in the library's layout;
    pin=True gives pinned host pools (device must be "cpu")."""
    es = torch.empty((), dtype=dtype).element_size()
    x = 16 // es
    kw = {"pin_memory": True} if pin else {}
    kc = torch.empty((num_blocks, num_kv_heads, head_dim // x, block_size, x), dtype=dtype,
                     device=device, **kw)
    vc = torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=dtype, device=device,
                     **kw)
    return kc, vc


def paged_kv_write(key, value, key_cache, value_cache, slot_mapping, k_scale=1.0, v_scale=1.0,
                   stream=None):
    nb, H, D, bs = _pool_shape(key_cache, value_cache)
    for t, n in ((key, "key"), (value, "value"), (key_cache, "key_cache"), (value_cache, "value_cache")):
        _need(t, n)
    _need(slot_mapping, "slot_mapping", torch.int32)
    T = key.shape[0]
    if tuple(key.shape) != (T, H, D) or tuple(value.shape) != (T, H, D) or slot_mapping.numel() != T:
        raise PkvError(-1, "key/value must be [T, H_kv, head_dim] with T slots")
    check(lib().paged_kv_write(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                               _ptr(slot_mapping), T, H, D, bs, nb, cache_dtype_code(key),
                               cache_dtype_code(key_cache), float(k_scale), float(v_scale),
                               _stream(stream)))


def paged_attention_partition_offsets(context_lens_host, partition_tokens: int):
    """Host-side partition offsets: (int32 numpy [S+1], total partitions)."""
    lens = np.ascontiguousarray(np.asarray(context_lens_host, dtype=np.int32))
    S = lens.size
    off = np.zeros(S + 1, dtype=np.int32)
    tot = ctypes.c_int(0)
    check(lib().paged_attention_partition_offsets(
        lens.ctypes.data_as(_native.pi32), S, int(partition_tokens),
        off.ctypes.data_as(_native.pi32), ctypes.byref(tot)))
    return off, tot.value


def paged_attention_workspace_bytes(total_partitions: int, num_q_heads: int, head_dim: int) -> int:
    return int(lib().paged_attention_workspace_bytes(total_partitions, num_q_heads, head_dim))


def _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale, k_scale,
                 v_scale, partition_tokens, partition_offsets, total_partitions, workspace):
    nb, H, D, bs = _pool_shape(key_cache, value_cache)
    for t, n in ((out, "out"), (query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache")):
        _need(t, n)
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32)
    S, Hq, Dq = query.shape
    if Dq != D or tuple(out.shape) != (S, Hq, D) or out.dtype != query.dtype:
        raise PkvError(-1, "query/out must be [S, H_q, head_dim] of one dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise PkvError(-1, "block_tables must be [S, max_blocks] and context_lens [S]")
    ws_bytes = 0
    if partition_tokens:
        if partition_offsets is None or workspace is None:
            raise PkvError(-3, "split-K needs partition_offsets and a workspace")
        _need(partition_offsets, "partition_offsets", torch.int32)
        _need(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    return (_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), S, Hq, H, D, bs, nb, float(scale),
            cache_dtype_code(query), cache_dtype_code(key_cache), float(k_scale), float(v_scale),
            int(partition_tokens), _ptr(partition_offsets), int(total_partitions), _ptr(workspace),
            ws_bytes)


def paged_attention_decode(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                           k_scale=1.0, v_scale=1.0, partition_tokens=0, partition_offsets=None,
                           total_partitions=0, workspace=None, stream=None):
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                        k_scale, v_scale, partition_tokens, partition_offsets, total_partitions,
                        workspace)
    check(lib().paged_attention_decode(*args, _stream(stream)))


def paged_attention_decode_noalloc(out, query, key_cache, value_cache, block_tables, context_lens,
                                   scale, k_scale=1.0, v_scale=1.0, partition_tokens=0,
                                   partition_offsets=None, total_partitions=0, stream=None):
    """paged_attention_decode with the split-K partials in the library's own
    static device array (PKV_NOALLOC_WORKSPACE_BYTES per GPU): no workspace
    argument, nothing allocated.  Calls that overlap on one GPU race."""
    nb, H, D, bs = _pool_shape(key_cache, value_cache)
    for t, n in ((out, "out"), (query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache")):
        _need(t, n)
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32)
    S, Hq, Dq = query.shape
    if Dq != D or tuple(out.shape) != (S, Hq, D) or out.dtype != query.dtype:
        raise PkvError(-1, "query/out must be [S, H_q, head_dim] of one dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise PkvError(-1, "block_tables must be [S, max_blocks] and context_lens [S]")
    if partition_tokens:
        if partition_offsets is None:
            raise PkvError(-1, "split-K needs partition_offsets")
        _need(partition_offsets, "partition_offsets", torch.int32)
    check(lib().paged_attention_decode_noalloc(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), S, Hq, H, D, bs, nb, float(scale),
        cache_dtype_code(query), cache_dtype_code(key_cache), float(k_scale), float(v_scale),
        int(partition_tokens), _ptr(partition_offsets), int(total_partitions), _stream(stream)))


def paged_attention_decode_queue(out, query, key_cache, value_cache, block_tables, context_lens,
                                 scale, k_scale=1.0, v_scale=1.0, partition_tokens=0,
                                 partition_offsets=None, total_partitions=0, workspace=None,
                                 stream=None):
    """paged_attention_decode's split-K with items handed out by a device
    work counter (fp8 matrix-core shape only; same result bit for bit)."""
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                        k_scale, v_scale, partition_tokens, partition_offsets, total_partitions,
                        workspace)
    check(lib().paged_attention_decode_queue(*args, _stream(stream)))


def paged_attention_decode_partials(out, query, key_cache, value_cache, block_tables, context_lens,
                                    scale, k_scale=1.0, v_scale=1.0, partition_tokens=0,
                                    partition_offsets=None, total_partitions=0, workspace=None,
                                    stream=None):
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                        k_scale, v_scale, partition_tokens, partition_offsets, total_partitions,
                        workspace)
    check(lib().paged_attention_decode_partials(*args, _stream(stream)))


def paged_attention_decode_step(out, query, new_key, new_value, key_cache, value_cache,
                                block_tables, context_lens, scale, k_scale=1.0, v_scale=1.0,
                                partition_tokens=0, partition_offsets=None, total_partitions=0,
                                workspace=None, stream=None):
    """Store each sequence's new key/value row (position context_lens[s]-1),
    then decode, as paged_kv_write followed by paged_attention_decode."""
    a = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                     k_scale, v_scale, partition_tokens, partition_offsets, total_partitions,
                     workspace)
    S, Hq, D = query.shape
    H = key_cache.shape[1]
    for t, n in ((new_key, "new_key"), (new_value, "new_value")):
        _need(t, n)
        if tuple(t.shape) != (S, H, D) or t.dtype != query.dtype:
            raise PkvError(-1, f"{n} must be [S, H_kv, head_dim] of the query dtype")
    check(lib().paged_attention_decode_step(a[0], a[1], _ptr(new_key), _ptr(new_value), *a[2:],
                                            _stream(stream)))


def paged_attention_decode_step_launches(num_q_heads, num_kv_heads, head_dim, block_size, q_dtype,
                                         cache_dtype, partition_tokens=0) -> int:
    """Kernel launches one decode step makes for this shape (1 = store inside the decode).
    Dtypes are torch dtypes (torch.uint8 for an FP8 cache) or pkv_dtype codes."""
    n = lib().paged_attention_decode_step_launches(num_q_heads, num_kv_heads, head_dim, block_size,
                                                   _dtype_code(q_dtype), _dtype_code(cache_dtype),
                                                   int(partition_tokens))
    check(min(n, 0))
    return n


def paged_attention_tile_offsets(context_lens_host, block_size: int):
    """Host-side stream-K tile offsets: (int32 numpy [S+1], total tiles)."""
    lens = np.ascontiguousarray(np.asarray(context_lens_host, dtype=np.int32))
    S = lens.size
    off = np.zeros(S + 1, dtype=np.int32)
    tot = ctypes.c_int(0)
    check(lib().paged_attention_tile_offsets(lens.ctypes.data_as(_native.pi32), S, int(block_size),
                                             off.ctypes.data_as(_native.pi32), ctypes.byref(tot)))
    return off, tot.value


def _dtype_code(t):
    if isinstance(t, int):
        return t
    if t not in _CODES:
        raise PkvError(-1, f"unsupported dtype {t}")
    return _CODES[t]


def paged_attention_streamk_workers(num_q_heads, num_kv_heads, head_dim, block_size, q_dtype,
                                    cache_dtype) -> int:
    n = lib().paged_attention_streamk_workers(num_q_heads, num_kv_heads, head_dim, block_size,
                                              _dtype_code(q_dtype), _dtype_code(cache_dtype))
    check(min(n, 0))
    return n


def paged_attention_streamk_workspace_bytes(workers, num_seqs, num_q_heads, num_kv_heads,
                                            head_dim) -> int:
    return int(lib().paged_attention_streamk_workspace_bytes(workers, num_seqs, num_q_heads,
                                                             num_kv_heads, head_dim))


def _streamk_args(query, key_cache, block_tables, context_lens, tile_offsets, total_tiles, workers,
                  workspace):
    _need(tile_offsets, "tile_offsets", torch.int32)
    _need(workspace, "workspace")
    S = query.shape[0]
    if tile_offsets.numel() != S + 1:
        raise PkvError(-1, "tile_offsets must have S + 1 entries")
    return (_ptr(tile_offsets), int(total_tiles)), (int(workers), _ptr(workspace),
                                                    workspace.numel() * workspace.element_size())


def paged_attention_decode_streamk(out, query, key_cache, value_cache, block_tables, context_lens,
                                   scale, tile_offsets, total_tiles, workers, workspace,
                                   k_scale=1.0, v_scale=1.0, stream=None):
    a = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                     k_scale, v_scale, 0, None, 0, None)
    mid, tail = _streamk_args(query, key_cache, block_tables, context_lens, tile_offsets,
                              total_tiles, workers, workspace)
    # a = (out, q, kc, vc, tables, max_blocks, lens, S, Hq, Hkv, D, bs, nb, scale, qdt, cdt,
    #      k_scale, v_scale, partition, part_off, total_parts, ws, ws_bytes)
    check(lib().paged_attention_decode_streamk(*a[:7], *mid, *a[7:18], *tail, _stream(stream)))


def paged_attention_decode_streamk_partials(out, query, key_cache, value_cache, block_tables,
                                            context_lens, scale, tile_offsets, total_tiles,
                                            workers, workspace, k_scale=1.0, v_scale=1.0,
                                            stream=None):
    a = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                     k_scale, v_scale, 0, None, 0, None)
    mid, tail = _streamk_args(query, key_cache, block_tables, context_lens, tile_offsets,
                              total_tiles, workers, workspace)
    check(lib().paged_attention_decode_streamk_partials(*a[:7], *mid, *a[7:18], *tail,
                                                        _stream(stream)))


def paged_attention_streamk_reduce(out, workspace, tile_offsets, total_tiles, workers,
                                   num_kv_heads, block_size, cache_dtype, stream=None):
    _need(out, "out")
    _need(workspace, "workspace")
    _need(tile_offsets, "tile_offsets", torch.int32)
    S, Hq, D = out.shape
    check(lib().paged_attention_streamk_reduce(
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(tile_offsets), int(total_tiles), S, Hq, int(num_kv_heads), D, int(block_size),
        cache_dtype_code(out), _dtype_code(cache_dtype), int(workers), _stream(stream)))


def paged_attention_decode_step_streamk(out, query, new_key, new_value, key_cache, value_cache,
                                        block_tables, context_lens, scale, tile_offsets,
                                        total_tiles, workers, workspace, k_scale=1.0, v_scale=1.0,
                                        stream=None):
    a = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                     k_scale, v_scale, 0, None, 0, None)
    S, Hq, D = query.shape
    H = key_cache.shape[1]
    for t, n in ((new_key, "new_key"), (new_value, "new_value")):
        _need(t, n)
        if tuple(t.shape) != (S, H, D) or t.dtype != query.dtype:
            raise PkvError(-1, f"{n} must be [S, H_kv, head_dim] of the query dtype")
    mid, tail = _streamk_args(query, key_cache, block_tables, context_lens, tile_offsets,
                              total_tiles, workers, workspace)
    check(lib().paged_attention_decode_step_streamk(a[0], a[1], _ptr(new_key), _ptr(new_value),
                                                    *a[2:7], *mid, *a[7:18], *tail,
                                                    _stream(stream)))


def paged_attention_prefix_plan(context_lens_host, group_offsets, group_prefix_blocks, block_size,
                                partition_tokens, num_q_heads, num_kv_heads):
    """Host plan of the shared-prefix decode: groups of consecutive sequences
    group_offsets[g] .. group_offsets[g+1] share their first
    group_prefix_blocks[g] blocks.  Returns a dict of int32 numpy arrays
    (row_offsets, suffix_offsets, token_start, prefix_item_offsets) and the
    totals (rows, suffix_partitions, prefix_items)."""
    lens = np.ascontiguousarray(np.asarray(context_lens_host, dtype=np.int32))
    go = np.ascontiguousarray(np.asarray(group_offsets, dtype=np.int32))
    gb = np.ascontiguousarray(np.asarray(group_prefix_blocks, dtype=np.int32))
    S, G = lens.size, gb.size
    if go.size != G + 1:
        raise PkvError(-1, "group_offsets must have one entry more than group_prefix_blocks")
    row = np.zeros(S + 1, np.int32)
    suf = np.zeros(S + 1, np.int32)
    ts = np.zeros(max(S, 1), np.int32)
    pre = np.zeros(G + 1, np.int32)
    tot = np.zeros(3, np.int32)
    P = lambda x: x.ctypes.data_as(_native.pi32)
    check(lib().paged_attention_prefix_plan(P(lens), S, P(go), P(gb), G, int(block_size),
                                            int(partition_tokens), int(num_q_heads),
                                            int(num_kv_heads), P(row), P(suf), P(ts), P(pre),
                                            P(tot)))
    return {"row_offsets": row, "suffix_offsets": suf, "token_start": ts[:S],
            "prefix_item_offsets": pre, "group_offsets": go, "group_prefix_blocks": gb,
            "totals": tuple(int(t) for t in tot)}


def _prefix_args(plan_dev, totals, workspace):
    names = ("group_offsets", "group_prefix_blocks", "row_offsets", "suffix_offsets",
             "token_start", "prefix_item_offsets")
    for n in names:
        _need(plan_dev[n], n, torch.int32)
    _need(workspace, "workspace")
    d = {n: _ptr(plan_dev[n]) for n in names}
    n_groups = plan_dev["group_prefix_blocks"].numel()
    return (d["group_offsets"], d["group_prefix_blocks"], n_groups, d["row_offsets"],
            d["suffix_offsets"], d["token_start"], d["prefix_item_offsets"], int(totals[0]),
            int(totals[1]), int(totals[2]), _ptr(workspace),
            workspace.numel() * workspace.element_size())


def paged_attention_decode_prefix(out, query, key_cache, value_cache, block_tables, context_lens,
                                  scale, partition_tokens, plan_dev, totals, workspace,
                                  k_scale=1.0, v_scale=1.0, stream=None):
    """Decode with each group's shared prefix blocks read once per 32 query
    rows.  plan_dev: device int32 tensors of the plan (group_offsets,
    group_prefix_blocks, row_offsets, suffix_offsets, token_start,
    prefix_item_offsets); totals: the plan's host totals."""
    a = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                     k_scale, v_scale, 0, None, 0, None)
    check(lib().paged_attention_decode_prefix(
        *a[:18], int(partition_tokens), *_prefix_args(plan_dev, totals, workspace),
        _stream(stream)))


def paged_attention_decode_prefix_step(out, query, new_key, new_value, key_cache, value_cache,
                                       block_tables, context_lens, scale, partition_tokens,
                                       plan_dev, totals, workspace, k_scale=1.0, v_scale=1.0,
                                       stream=None):
    """Store each sequence's new key/value row (position context_lens[s]-1),
    then decode with the shared-prefix schedule, as paged_kv_write followed by
    paged_attention_decode_prefix; the plan is the step's (new token
    included)."""
    a = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                     k_scale, v_scale, 0, None, 0, None)
    S, Hq, D = query.shape
    H = key_cache.shape[1]
    for t, n in ((new_key, "new_key"), (new_value, "new_value")):
        _need(t, n)
        if tuple(t.shape) != (S, H, D) or t.dtype != query.dtype:
            raise PkvError(-1, f"{n} must be [S, H_kv, head_dim] of the query dtype")
    check(lib().paged_attention_decode_prefix_step(
        a[0], a[1], _ptr(new_key), _ptr(new_value), *a[2:18], int(partition_tokens),
        *_prefix_args(plan_dev, totals, workspace), _stream(stream)))


def paged_attention_prefill(out, query, key_cache, value_cache, block_tables, context_lens,
                            query_start, max_query_len, scale, k_scale=1.0, v_scale=1.0,
                            stream=None):
    """Chunked prefill: query rows [T, H_q, head_dim] of every sequence's last
    C_s positions (C_s = query_start[s+1] - query_start[s]), causal attention
    over the paged cache into out [T, H_q, head_dim]."""
    nb, H, D, bs = _pool_shape(key_cache, value_cache)
    for t, n in ((out, "out"), (query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache")):
        _need(t, n)
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32)
    _need(query_start, "query_start", torch.int32)
    T, Hq, Dq = query.shape
    S = context_lens.numel()
    if Dq != D or tuple(out.shape) != (T, Hq, D) or out.dtype != query.dtype:
        raise PkvError(-1, "query/out must be [T, H_q, head_dim] of one dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start.numel() != S + 1:
        raise PkvError(-1, "block_tables must be [S, max_blocks] and query_start [S + 1]")
    check(lib().paged_attention_prefill(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(query_start), S, int(max_query_len), Hq,
        H, D, bs, nb, float(scale), cache_dtype_code(query), cache_dtype_code(key_cache),
        float(k_scale), float(v_scale), _stream(stream)))


def paged_attention_splitk_reduce(out, workspace, partition_offsets, total_partitions,
                                  max_partitions_per_seq=0, stream=None):
    _need(out, "out")
    _need(workspace, "workspace")
    _need(partition_offsets, "partition_offsets", torch.int32)
    S, Hq, D = out.shape
    check(lib().paged_attention_splitk_reduce(
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(partition_offsets), S, Hq, D, int(total_partitions), int(max_partitions_per_seq),
        cache_dtype_code(out), _stream(stream)))


def paged_kv_copy_blocks(key_cache, value_cache, pairs, stream=None):
    nb, H, D, bs = _pool_shape(key_cache, value_cache)
    _need(key_cache, "key_cache")
    _need(value_cache, "value_cache")
    _need(pairs, "pairs", torch.int32)
    n = pairs.numel() // 2
    block_bytes = H * bs * D * key_cache.element_size()
    check(lib().paged_kv_copy_blocks(_ptr(key_cache), _ptr(value_cache), _ptr(pairs), n,
                                     block_bytes, nb, _stream(stream)))


def host_device_pointer(t: torch.Tensor) -> int:
    """Device pointer of a pinned host tensor (the library refuses memory
    that is not pinned)."""
    if t.is_cuda or not t.is_pinned():
        raise PkvError(-1, "expected a pinned host tensor")
    out = ctypes.c_void_p()
    check(lib().pkv_host_device_pointer(ctypes.c_void_p(t.data_ptr()), ctypes.byref(out)))
    return int(out.value)


def _pool_ptr(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise PkvError(-1, f"{name} must be contiguous")
    if t.is_cuda:
        return ctypes.c_void_p(t.data_ptr())
    return ctypes.c_void_p(host_device_pointer(t))


def paged_kv_swap_blocks(dst_key, dst_value, src_key, src_value, pairs, stream=None):
    """Copy whole blocks src block p[0] -> dst block p[1] for each pair,
    between a device pool and a pinned host pool of the same layout."""
    nbs, H, D, bs = _pool_shape(src_key, src_value)
    nbd, Hd, Dd, bsd = _pool_shape(dst_key, dst_value)
    if (H, D, bs) != (Hd, Dd, bsd) or src_key.dtype != dst_key.dtype:
        raise PkvError(-1, "source and destination pools differ in layout")
    _need(pairs, "pairs", torch.int32)
    block_bytes = H * bs * D * src_key.element_size()
    check(lib().paged_kv_swap_blocks(
        _pool_ptr(dst_key, "dst_key"), _pool_ptr(dst_value, "dst_value"),
        _pool_ptr(src_key, "src_key"), _pool_ptr(src_value, "src_value"), _ptr(pairs),
        pairs.numel() // 2, block_bytes, nbs, nbd, _stream(stream)))


def paged_kv_swap_blocks_memcpy(dst_key, dst_value, src_key, src_value, pairs, stream=None):
    """paged_kv_swap_blocks as asynchronous copies: pairs is a host int32
    array [n][2]; each run of consecutive (src, dst) ids is one
    hipMemcpyAsync per pool on `stream`."""
    nbs, H, D, bs = _pool_shape(src_key, src_value)
    nbd, Hd, Dd, bsd = _pool_shape(dst_key, dst_value)
    if (H, D, bs) != (Hd, Dd, bsd) or src_key.dtype != dst_key.dtype:
        raise PkvError(-1, "source and destination pools differ in layout")
    p = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    block_bytes = H * bs * D * src_key.element_size()
    check(lib().paged_kv_swap_blocks_memcpy(
        _pool_ptr(dst_key, "dst_key"), _pool_ptr(dst_value, "dst_value"),
        _pool_ptr(src_key, "src_key"), _pool_ptr(src_value, "src_value"),
        p.ctypes.data_as(_native.pi32), p.shape[0], block_bytes, nbs, nbd, _stream(stream)))


def pkv_paged_read_probe(key_cache, value_cache, block_tables, context_lens, num_q_heads, q_dtype,
                         partition_tokens, partition_offsets, total_partitions, sink, stream=None):
    """The split-K decode's reads alone (measurement aid); sink: device tensor
    of >= 4 bytes, 16-byte aligned."""
    nb, H, D, bs = _pool_shape(key_cache, value_cache)
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32)
    _need(partition_offsets, "partition_offsets", torch.int32)
    _need(sink, "sink")
    check(lib().pkv_paged_read_probe(
        _ptr(key_cache), _ptr(value_cache), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), context_lens.numel(), int(num_q_heads), H, D, bs, nb,
        _CODES[q_dtype], cache_dtype_code(key_cache), int(partition_tokens),
        _ptr(partition_offsets), int(total_partitions), _ptr(sink), _stream(stream)))


def paged_kv_gather(k_out, v_out, key_cache, value_cache, block_tables, cu_ctx, total_tokens,
                    stream=None):
    nb, H, D, bs = _pool_shape(key_cache, value_cache)
    for t, n in ((k_out, "k_out"), (v_out, "v_out"), (key_cache, "key_cache"), (value_cache, "value_cache")):
        _need(t, n)
    _need(block_tables, "block_tables", torch.int32)
    _need(cu_ctx, "cu_ctx", torch.int32)
    if tuple(k_out.shape) != (total_tokens, H, D) or tuple(v_out.shape) != (total_tokens, H, D):
        raise PkvError(-1, "k_out/v_out must be [total_tokens, H_kv, head_dim]")
    S = cu_ctx.numel() - 1
    check(lib().paged_kv_gather(_ptr(k_out), _ptr(v_out), _ptr(key_cache), _ptr(value_cache),
                                _ptr(block_tables), block_tables.shape[1], _ptr(cu_ctx), S,
                                int(total_tokens), H, D, bs, nb, cache_dtype_code(key_cache),
                                _stream(stream)))


def pkv_hbm_read_probe(buffer: torch.Tensor, sink: torch.Tensor, workgroups: int, stream=None):
    """Stream-read the whole of `buffer` (device); see include/pkv.h."""
    _need(buffer, "buffer")
    _need(sink, "sink")
    check(lib().pkv_hbm_read_probe(_ptr(buffer), buffer.numel() * buffer.element_size(),
                                   _ptr(sink), int(workgroups), _stream(stream)))


class BlockAllocator:
    """Host block allocator of libpkv (pkv_alloc_*); not thread-safe."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        fo = None
        if free_order is not None:
            self._fo = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if self._fo.size != num_blocks:
                raise PkvError(-1, "free_order must have num_blocks entries")
            fo = self._fo.ctypes.data_as(_native.pi32)
        h = lib().pkv_alloc_create(int(num_blocks), int(block_size), fo)
        if not h:
            raise PkvError(-1, lib().pkv_last_error().decode())
        self._h = ctypes.c_void_p(h)

    def close(self):
        if getattr(self, "_h", None):
            lib().pkv_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_seq(self, seq: int):
        check(lib().pkv_alloc_add_seq(self._h, int(seq)))

    def fork(self, parent: int, child: int):
        check(lib().pkv_alloc_fork(self._h, int(parent), int(child)))

    def append(self, seq: int, n: int):
        """Returns (slots int32 [n], cow pairs int32 [k, 2])."""
        slots = np.zeros(max(int(n), 1), dtype=np.int32)
        cow = np.zeros(2, dtype=np.int32)
        ncow = ctypes.c_int(0)
        check(lib().pkv_alloc_append(self._h, int(seq), int(n), slots.ctypes.data_as(_native.pi32),
                                     cow.ctypes.data_as(_native.pi32), 1, ctypes.byref(ncow)))
        return slots[:int(n)], cow[:2 * ncow.value].reshape(-1, 2)

    def free_seq(self, seq: int):
        check(lib().pkv_alloc_free_seq(self._h, int(seq)))

    def seq_len(self, seq: int) -> int:
        r = lib().pkv_alloc_len(self._h, int(seq))
        if r < 0:
            check(int(r))
        return int(r)

    def block_table(self, seq: int) -> np.ndarray:
        cap = self.seq_len(seq) // self.block_size + 1
        out = np.zeros(cap, dtype=np.int32)
        n = ctypes.c_int(0)
        check(lib().pkv_alloc_block_table(self._h, int(seq), out.ctypes.data_as(_native.pi32), cap,
                                          ctypes.byref(n)))
        return out[:n.value]

    def fill_tables(self, seqs, width: int, pad: int = -1) -> np.ndarray:
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        out = np.zeros((seqs.size, int(width)), dtype=np.int32)
        check(lib().pkv_alloc_fill_tables(self._h, seqs.ctypes.data_as(_native.pi64), seqs.size,
                                          out.ctypes.data_as(_native.pi32), int(width), int(pad)))
        return out

    def refcount(self, block: int) -> int:
        return check_nonneg(lib().pkv_alloc_refcount(self._h, int(block)))

    def num_free(self) -> int:
        return check_nonneg(lib().pkv_alloc_num_free(self._h))

    def free_list(self) -> list:
        out = np.zeros(self.num_blocks, dtype=np.int32)
        n = lib().pkv_alloc_free_list(self._h, out.ctypes.data_as(_native.pi32), self.num_blocks)
        return [int(b) for b in out[:check_nonneg(n)]]

    def set_host_pool(self, num_host_blocks: int):
        check(lib().pkv_alloc_set_host_pool(self._h, int(num_host_blocks)))

    def _swap(self, fn, seq):
        cap = self.seq_len(seq) // self.block_size + 1
        out = np.zeros(2 * cap, dtype=np.int32)
        n = ctypes.c_int(0)
        check(fn(self._h, int(seq), out.ctypes.data_as(_native.pi32), cap, ctypes.byref(n)))
        return [(int(out[2 * i]), int(out[2 * i + 1])) for i in range(n.value)]

    def swap_out(self, seq: int) -> list:
        """Pairs (device block, host slot), one per table entry."""
        return self._swap(lib().pkv_alloc_swap_out, seq)

    def swap_in(self, seq: int) -> list:
        """Pairs (host slot, device block), one per table entry."""
        return self._swap(lib().pkv_alloc_swap_in, seq)

    def touch(self, seq: int):
        check(lib().pkv_alloc_touch(self._h, int(seq)))

    def lru(self) -> int:
        out = ctypes.c_int64(0)
        check(lib().pkv_alloc_lru(self._h, ctypes.byref(out)))
        return int(out.value)

    def lfu(self) -> int:
        out = ctypes.c_int64(0)
        check(lib().pkv_alloc_lfu(self._h, ctypes.byref(out)))
        return int(out.value)

    def is_swapped(self, seq: int) -> bool:
        return bool(check_nonneg(lib().pkv_alloc_is_swapped(self._h, int(seq))))

    def num_host_free(self) -> int:
        return check_nonneg(lib().pkv_alloc_num_host_free(self._h))


def check_nonneg(r: int) -> int:
    if r < 0:
        check(r)
    return r
