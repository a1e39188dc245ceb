"""Loads a workload description onto the device through the library's own
allocator, copy and write calls (the HIP side of a test or of the bench; the
oracle side never imports this module, and it does none of the method's
arithmetic: it orders calls to the C ABI).

A workload is any object with ``cfg`` (S, H_kv, d, bs, dtypes, fp8 scales),
``num_blocks``, ``free_order``, ``q`` (query bits), ``prefill`` / ``decode``
operation lists of ("add", s), ("fork", parent, child) and
("append", s, n, stream, start), and ``values(stream, start, n)`` returning
the stored bits of the appended key and value rows.
"""

from __future__ import annotations

import numpy as np
import torch

TORCH_CACHE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
# a byte whose repetition is NaN in every cache format: fp32 0xFFFFFFFF, bf16
# 0xFFFF, fp8 0xFF (S.1111.111)
POISON_BYTE = 0xFF


def to_dev(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
    raise ValueError(dtype)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _flush(cache, items):
    if items:
        cache.append_many(items)
        items.clear()


def run_ops(cache, wl, ops, device="cuda", flush_tokens=1 << 22):
    c = wl.cfg
    items, pending = [], 0
    for op in ops:
        if op[0] == "add":
            cache.add_seq(op[1])
        elif op[0] == "fork":
            _flush(cache, items)
            pending = 0
            cache.fork(op[1], op[2])
        else:
            _, s, n, stream, start = op
            k, v = wl.values(stream, start, n)
            items.append((s, to_dev(k, c.src_dtype, device), to_dev(v, c.src_dtype, device)))
            pending += n
            if pending >= flush_tokens:
                _flush(cache, items)
                pending = 0
    _flush(cache, items)


def build(wl, poison=True, device="cuda", write_step=True):
    """Prefill through the library, then allocate and write the decode step
    (write_step=False: allocate it only, for a fused step to store).

    Returns (cache, step) where step holds the decode-step slot mapping and
    new key/value rows (device, row s = sequence s) and the query.
    """
    from paged_kv_cache_211_amd.engine import PagedKVCache
    c = wl.cfg
    cache = PagedKVCache(wl.num_blocks, c.H_kv, c.d, c.bs, TORCH_CACHE[c.kv_dtype], device,
                         free_order=wl.free_order, k_scale=c.k_scale, v_scale=c.v_scale,
                         fill_byte=POISON_BYTE if poison else 0)
    run_ops(cache, wl, wl.prefill, device)
    # decode step: one token per sequence, written with a single call
    ks, vs = [], []
    for op in wl.decode:
        _, s, n, stream, start = op
        k, v = wl.values(stream, start, n)
        ks.append(k)
        vs.append(v)
    K = to_dev(np.concatenate(ks), c.src_dtype, device)
    V = to_dev(np.concatenate(vs), c.src_dtype, device)
    assert [op[1] for op in wl.decode] == list(range(len(wl.decode))), "one token per sequence, in order"
    items = [(op[1], K[i:i + 1], V[i:i + 1]) for i, op in enumerate(wl.decode)]
    slots = cache.append_many(items, write=write_step)
    step = {"slots": slots, "slots_dev": torch.from_numpy(slots).to(device), "key": K, "value": V,
            "query": to_dev(wl.q, c.q_dtype, device)}
    return cache, step
