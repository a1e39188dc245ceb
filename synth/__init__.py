"""Seeded synthetic workloads for PagedAttention decode.

This module only draws random inputs and describes the sequence of allocator
operations a workload performs; it holds none of the method's arithmetic
(no slot computation, no layout, no attention).  Both the oracle side and the
HIP side of a test consume exactly what it returns, each through its own
allocator, scatter and attention.

Recipe (per workload, seed ``seed``):
  * context lengths from ``numpy.random.default_rng(seed)`` (integer uniform,
    bounds inclusive), then the pool's free order as a permutation of the
    physical block ids from the same generator;
  * queries from ``default_rng([seed, 1])``: fp32 N(0, 1) rounded to nearest
    even into the query dtype;
  * the keys and values of sequence s's own tokens from
    ``default_rng([seed, 2, s])`` (keys drawn first, then values), and those
    of a shared prompt prefix from ``default_rng([seed, 3])``: fp32 N(0, 1)
    rounded to nearest even into the written dtype (bf16 also for an fp8
    cache, which quantises on write with fixed per-tensor scales: 8/448 for
    keys and for values in the full-size workload, i.e. +-8 standard
    deviations map to the largest finite E4M3FN value; the small skewed
    workload keeps 8/448 for keys and takes 2/448 for values, so that
    routing one pool's scale to the other changes every output by a factor
    of about four and the parity tests see it).

Operations: every sequence is added, prefilled with all but its last token,
and then one decode step appends exactly one token per sequence, so the
context length of the step counts the token written in that step.  A shared
prefix is prefilled once on sequence 0, forked to every other sequence, and
each sequence then appends its private suffix in sequence order.

Chunked prefill inputs (``PREFILL``): the same cache recipe, then each
sequence's last C_s tokens are taken as the chunk whose query rows attend
over the cache; chunk lengths from ``default_rng([seed, 6])`` (integer
uniform over [lo, hi] clipped to the context), chunk query rows from
``default_rng([seed, 5])`` as fp32 N(0, 1) rounded into the query dtype.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}
FP8_KV_SCALE = float(np.float32(8.0 / 448.0))
FP8_V_SCALE_SMALL = float(np.float32(2.0 / 448.0))


@dataclass(frozen=True)
class Config:
    key: str
    S: int
    H_q: int
    H_kv: int
    d: int
    bs: int
    q_dtype: str           # "f32" | "bf16"
    kv_dtype: str          # cache storage: "f32" | "bf16" | "fp8"
    scale: float           # softmax scale, an fp32 value
    partition: int         # split-K partition length (tokens) used at launch; 0 = one pass
    seed: int
    lens: tuple = ()       # fixed context lengths, or
    len_range: tuple = ()  # (lo, hi) inclusive uniform
    long: tuple = ()       # (count, lo, hi) long sequences first ...
    short: tuple = ()      # ... then (count, lo, hi) short ones
    prefix: int = 0        # shared prompt prefix length (tokens)
    suffix_range: tuple = ()
    chunk: tuple = ()      # chunked prefill: (lo, hi) query rows per sequence
    num_blocks: int = 0    # fixed pool size; 0 = two times the blocks the workload needs
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def src_dtype(self) -> str:
        """dtype of the key/value rows handed to the write."""
        return "f32" if self.kv_dtype == "f32" else "bf16"

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv


_SCALE_D128 = float(np.float32(1.0 / math.sqrt(128.0)))

# `partition` is the split-K length the launches use: the specified one
# where a workload names it (the skewed fp8 workload: 512 tokens), else the
# fastest measured.
CONFIGS = {
    1: Config("fp32-tiny", S=4, H_q=4, H_kv=4, d=64, bs=16, q_dtype="f32", kv_dtype="f32",
              scale=0.125, partition=0, seed=1, lens=(1, 17, 33, 100), num_blocks=64),
    2: Config("bf16-mha-7b", S=32, H_q=32, H_kv=32, d=128, bs=16, q_dtype="bf16", kv_dtype="bf16",
              scale=_SCALE_D128, partition=256, seed=2, len_range=(128, 2048)),
    3: Config("bf16-gqa", S=64, H_q=32, H_kv=8, d=128, bs=16, q_dtype="bf16", kv_dtype="bf16",
              scale=_SCALE_D128, partition=1536, seed=3, len_range=(512, 8192)),
    4: Config("bf16-prefix", S=128, H_q=32, H_kv=8, d=128, bs=16, q_dtype="bf16", kv_dtype="bf16",
              scale=_SCALE_D128, partition=2048, seed=4, prefix=1030, suffix_range=(16, 512)),
    5: Config("fp8-skewed", S=256, H_q=64, H_kv=8, d=128, bs=32, q_dtype="bf16", kv_dtype="fp8",
              scale=_SCALE_D128, partition=512, seed=5, long=(8, 32768, 131072),
              short=(248, 64, 512), k_scale=FP8_KV_SCALE, v_scale=FP8_KV_SCALE),
}

# The same shapes, dtypes and structure at sizes a pure CPU oracle finishes in
# seconds; each still spans several blocks, several split-K partitions and a
# ragged last block.
SMALL = {
    1: replace(CONFIGS[1], key="fp32-tiny", seed=101),
    2: replace(CONFIGS[2], key="bf16-mha-small", S=5, partition=128, seed=102, len_range=(20, 300)),
    3: replace(CONFIGS[3], key="bf16-gqa-small", S=6, seed=103, len_range=(100, 1500),
               partition=512),
    4: replace(CONFIGS[4], key="bf16-prefix-small", S=8, seed=104, prefix=70, suffix_range=(5, 60),
               partition=64),
    5: replace(CONFIGS[5], key="fp8-skewed-small", S=8, seed=105, long=(2, 1500, 3000),
               short=(6, 10, 100), partition=512, v_scale=FP8_V_SCALE_SMALL),
}


# Chunked prefill over the paged cache: the GQA shape with each sequence's
# last 512 tokens as the chunk (full size), and small cases the oracle
# finishes in seconds (several blocks, several 32-row query blocks, ragged
# chunks from 1 row to the whole context).
PREFILL = {
    "full": Config("bf16-gqa-prefill", S=16, H_q=32, H_kv=8, d=128, bs=16, q_dtype="bf16",
                   kv_dtype="bf16", scale=_SCALE_D128, partition=0, seed=6,
                   len_range=(1024, 8192), chunk=(512, 512)),
    "small": Config("bf16-gqa-prefill-small", S=5, H_q=32, H_kv=8, d=128, bs=16, q_dtype="bf16",
                    kv_dtype="bf16", scale=_SCALE_D128, partition=0, seed=106,
                    len_range=(20, 300), chunk=(1, 120)),
}


def prefill_chunks(wl: "Workload", lo: int | None = None, hi: int | None = None) -> np.ndarray:
    """Seeded chunk lengths [S] (int64): C_s uniform in [min(lo, L_s), min(hi, L_s)]."""
    c = wl.cfg
    lo = c.chunk[0] if lo is None else lo
    hi = c.chunk[1] if hi is None else hi
    rng = np.random.default_rng([c.seed, 6])
    L = wl.context_lens
    return np.array([rng.integers(min(lo, int(l)), min(hi, int(l)), endpoint=True) for l in L],
                    dtype=np.int64)


def extra_rows(wl: "Workload", n: int, tag: int):
    """Seeded key/value rows [n, H_kv, d] (stored bits of the written dtype)
    for a sequence outside the workload, from default_rng([seed, 7, tag])."""
    c = wl.cfg
    rng = np.random.default_rng([c.seed, 7, tag])
    k = _round(rng.standard_normal((n, c.H_kv, c.d), dtype=np.float32), c.src_dtype)
    v = _round(rng.standard_normal((n, c.H_kv, c.d), dtype=np.float32), c.src_dtype)
    return k, v


def prefill_queries(wl: "Workload", chunk_lens) -> np.ndarray:
    """Seeded chunk query rows, stored bits [sum(chunk_lens), H_q, d]."""
    c = wl.cfg
    T = int(np.sum(chunk_lens))
    rng = np.random.default_rng([c.seed, 5])
    return _round(rng.standard_normal((T, c.H_q, c.d), dtype=np.float32), c.q_dtype)


def _round(x32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draws -> stored bits of ``dtype`` (round to nearest even)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


@dataclass
class Workload:
    cfg: Config
    context_lens: np.ndarray           # int64 [S], lengths after the decode step
    num_blocks: int
    free_order: np.ndarray             # int64 [num_blocks]
    q: np.ndarray                      # raw bits [S, H_q, d]
    prefill: list = field(default_factory=list)
    decode: list = field(default_factory=list)
    _cache: dict = field(default_factory=dict, repr=False)
    cache_limit: int = 4                # value streams kept in memory (0 = no limit)

    # ops are tuples:
    #   ("add", s)  ("fork", parent, child)
    #   ("append", s, n, stream, start)   stream = ("seq", s) | ("prefix",)

    def stream_len(self, stream) -> int:
        c = self.cfg
        if stream[0] == "prefix":
            return c.prefix
        return int(self.context_lens[stream[1]]) - c.prefix

    def stream(self, stream):
        """All key and value rows of one value stream, as stored bits."""
        if stream in self._cache:
            return self._cache[stream]
        c = self.cfg
        n = self.stream_len(stream)
        seed = [c.seed, 3] if stream[0] == "prefix" else [c.seed, 2, stream[1]]
        rng = np.random.default_rng(seed)
        k = _round(rng.standard_normal((n, c.H_kv, c.d), dtype=np.float32), c.src_dtype)
        v = _round(rng.standard_normal((n, c.H_kv, c.d), dtype=np.float32), c.src_dtype)
        if self.cache_limit and len(self._cache) >= self.cache_limit:
            self._cache.clear()
        self._cache[stream] = (k, v)
        return k, v

    def values(self, stream, start: int, n: int):
        k, v = self.stream(stream)
        return k[start:start + n], v[start:start + n]

    def drop_cache(self):
        self._cache.clear()

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.sum())


def _context_lens(c: Config, rng) -> np.ndarray:
    if c.lens:
        return np.array(c.lens, dtype=np.int64)
    if c.len_range:
        lo, hi = c.len_range
        return rng.integers(lo, hi, size=c.S, endpoint=True).astype(np.int64)
    if c.long:
        nl, llo, lhi = c.long
        ns, slo, shi = c.short
        assert nl + ns == c.S
        a = rng.integers(llo, lhi, size=nl, endpoint=True)
        b = rng.integers(slo, shi, size=ns, endpoint=True)
        return np.concatenate([a, b]).astype(np.int64)
    if c.prefix:
        lo, hi = c.suffix_range
        return (c.prefix + rng.integers(lo, hi, size=c.S, endpoint=True)).astype(np.int64)
    raise ValueError("config has no length recipe")


def _blocks_needed(c: Config, lens: np.ndarray) -> int:
    per_seq = (lens + c.bs - 1) // c.bs
    if not c.prefix:
        return int(per_seq.sum())
    shared_full = c.prefix // c.bs  # full prefix blocks stay shared
    return int(shared_full + (per_seq - shared_full).sum())


def make(cfg, seed: int | None = None) -> Workload:
    """Build the seeded workload for a config (a Config, or a key of CONFIGS)."""
    c = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    if seed is not None:
        c = replace(c, seed=seed)
    rng = np.random.default_rng(c.seed)
    lens = _context_lens(c, rng)
    assert (lens >= 1).all()
    nb = c.num_blocks or 2 * _blocks_needed(c, lens)
    free_order = rng.permutation(nb).astype(np.int64)
    qrng = np.random.default_rng([c.seed, 1])
    q = _round(qrng.standard_normal((c.S, c.H_q, c.d), dtype=np.float32), c.q_dtype)

    pre, dec = [], []
    if c.prefix:
        pre.append(("add", 0))
        pre.append(("append", 0, c.prefix, ("prefix",), 0))
        for s in range(1, c.S):
            pre.append(("fork", 0, s))
        for s in range(c.S):
            own = int(lens[s]) - c.prefix
            pre.append(("append", s, own - 1, ("seq", s), 0))
            dec.append(("append", s, 1, ("seq", s), own - 1))
    else:
        for s in range(c.S):
            pre.append(("add", s))
            pre.append(("append", s, int(lens[s]) - 1, ("seq", s), 0))
            dec.append(("append", s, 1, ("seq", s), int(lens[s]) - 1))
    return Workload(cfg=c, context_lens=lens, num_blocks=nb, free_order=free_order, q=q,
                    prefill=pre, decode=dec)


def private_copy(wl: Workload) -> Workload:
    """The same prefix workload with every sequence holding a private copy of
    the prefix instead of sharing it (same values, no fork)."""
    c = wl.cfg
    assert c.prefix
    pre, dec = [], []
    for s in range(c.S):
        own = int(wl.context_lens[s]) - c.prefix
        pre.append(("add", s))
        pre.append(("append", s, c.prefix, ("prefix",), 0))
        pre.append(("append", s, own - 1, ("seq", s), 0))
        dec.append(("append", s, 1, ("seq", s), own - 1))
    nb = 2 * int(((wl.context_lens + c.bs - 1) // c.bs).sum())
    rng = np.random.default_rng([c.seed, 4])
    return Workload(cfg=c, context_lens=wl.context_lens.copy(), num_blocks=nb,
                    free_order=rng.permutation(nb).astype(np.int64), q=wl.q.copy(),
                    prefill=pre, decode=dec)


def with_free_order(wl: Workload, free_order) -> Workload:
    """The same workload drawing physical blocks in another order."""
    return Workload(cfg=wl.cfg, context_lens=wl.context_lens.copy(), num_blocks=wl.num_blocks,
                    free_order=np.asarray(free_order, dtype=np.int64), q=wl.q.copy(),
                    prefill=list(wl.prefill), decode=list(wl.decode))
