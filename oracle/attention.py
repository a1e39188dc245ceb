"""Dense fp64 single-query softmax attention over a gathered cache (oracle).

PagedAttention changes where the cache lives, not what attention computes:
the block table makes a scattered cache read as if it were contiguous ("Day
6/90 of Inference Engineering", PagedAttention notes), and the kernel still
forms QK^T, normalises with softmax and accumulates PV, only block by block
("PagedAttention Kernel：大模型推理优化的显存管理革新" §3.1).  So the oracle is
the definition itself, in fp64, after gathering each sequence through its
table:

    z_t  = scale * sum_i q_i k_{t,i}                       t = 0 .. L-1
    w_t  = exp(z_t - max_u z_u) / sum_u exp(z_u - max_u z_u)
    out  = sum_t w_t v_t

Query head g of a group of G = H_q / H_kv heads reads kv head g // G (a
reading: the pages never mention grouped heads).  An empty context (L = 0)
returns zeros.  ``scale`` is taken as the exact fp32 value the kernel receives.

Chunked prefill (``paged_prefill``).  The pages only describe decode; the
plainest reading for a chunk of new tokens is ordinary causal attention over
the same contiguous view: sequence s holds L tokens whose last C are the
chunk, and chunk row i, at position p = L - C + i, attends tokens 0 .. p
(the tokens before it in the sequence and itself).  A chunk of one row is a
decode step.

Pins (tests/test_oracle_attention.py): torch's scaled_dot_product_attention
in fp64 on the contiguous (never paged) cache, with enable_gqa for grouped
heads; a pure-Python loop with math.fsum on tiny inputs; closed forms (L = 1
returns its value row, q = 0 returns the mean of the value rows, constant
value rows return the constant, two keys give the logistic weights); the
hand-computed example in tests/golden/attention_tiny.json; invariance under
any permutation of physical blocks and under prefix sharing.  For an fp8
cache: the SDPA pin quantises and dequantises with torch's own float8_e4m3fn
type (not this package's codec), on a workload with distinct key and value
scales; a hand-computed two-token case pins the key scale to the scores and
the value scale to the output (tests/test_oracle_fp8_scales.py).  Prefill pins
(tests/test_oracle_prefill.py): torch's scaled_dot_product_attention in fp64
with an explicit causal mask on the contiguous cache; a pure-Python fsum
evaluation on tiny paged inputs; q = 0 gives the running mean of the value
rows up to each position; a chunk's last row equals the decode output.
"""

from __future__ import annotations

import numpy as np

from .formats import decode
from .layout import gather_seq


def attend_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """One query row q [d] against keys K [L, d] and values V [L, d], in fp64.

    Returns (out [d], sum of the softmax weights).
    """
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1], dtype=np.float64), 0.0
    z = float(np.float32(scale)) * (K @ q)
    e = np.exp(z - z.max())
    w = e / e.sum()
    return w @ V, float(w.sum())


def dense_decode(q: np.ndarray, Ks, Vs, scale: float):
    """Decode attention for every sequence and query head.

    q  : fp64 [S, H_q, d]
    Ks : list of fp64 [L_s, H_kv, d] (token-major, contiguous) per sequence
    Vs : same for values
    Returns (out fp64 [S, H_q, d], weight sums fp64 [S, H_q]).
    """
    S, H_q, d = q.shape
    out = np.zeros((S, H_q, d), dtype=np.float64)
    wsum = np.zeros((S, H_q), dtype=np.float64)
    for s in range(S):
        H_kv = Ks[s].shape[1]
        G = H_q // H_kv
        for g in range(H_q):
            h = g // G
            out[s, g], wsum[s, g] = attend_one(q[s, g], Ks[s][:, h, :], Vs[s][:, h, :], scale)
    return out, wsum


def dequant(bits: np.ndarray, dtype: str, mult: float) -> np.ndarray:
    """Stored bits -> fp64 values; fp8 codes are multiplied by their scale."""
    v = decode(bits, dtype)
    if dtype == "fp8":
        v = v * float(np.float32(mult))  # exact: <=4-bit by 24-bit significands
    return v


def paged_decode(q_bits, q_dtype, kc, vc, block_tables, context_lens, *, bs, cache_dtype,
                 scale, k_scale=1.0, v_scale=1.0, seqs=None):
    """Gather every sequence through its block table, then attend in fp64.

    ``seqs`` restricts the work to a subset of sequence indices (the rest of
    the output stays zero); used to check sampled outputs of large batches.
    Returns (out [S, H_q, d], weight sums [S, H_q]).
    """
    q = decode(q_bits, q_dtype)
    S, H_q, d = q.shape
    out = np.zeros((S, H_q, d), dtype=np.float64)
    wsum = np.zeros((S, H_q), dtype=np.float64)
    todo = range(S) if seqs is None else seqs
    for s in todo:
        L = int(context_lens[s])
        kb, vb = gather_seq(kc, vc, block_tables[s], L, bs=bs)
        K = dequant(kb, cache_dtype, k_scale)
        V = dequant(vb, cache_dtype, v_scale)
        o, w = dense_decode(q[s:s + 1], [K], [V], scale)
        out[s], wsum[s] = o[0], w[0]
    return out, wsum


def paged_prefill(q_bits, q_dtype, kc, vc, block_tables, context_lens, query_start, *, bs,
                  cache_dtype, scale, k_scale=1.0, v_scale=1.0, seqs=None):
    """Causal attention of every sequence's chunk of query rows over its cache.

    q_bits      : stored bits [T, H_q, d], the chunks of all sequences in order
    query_start : [S + 1] row offsets; sequence s owns rows
                  query_start[s] .. query_start[s + 1] - 1, its last
                  C = query_start[s + 1] - query_start[s] <= context_lens[s]
                  positions
    ``seqs`` restricts the work to a subset of sequences (other rows stay 0).
    Returns out fp64 [T, H_q, d].

    Per (sequence, query head): Z = scale * Q K^T over the gathered keys, the
    entries of row i at positions t > L - C + i set to -inf, a row softmax,
    then times V.
    """
    q = decode(q_bits, q_dtype)
    T, H_q, d = q.shape
    out = np.zeros((T, H_q, d), dtype=np.float64)
    todo = range(len(context_lens)) if seqs is None else seqs
    sc = float(np.float32(scale))
    for s in todo:
        r0, r1 = int(query_start[s]), int(query_start[s + 1])
        C, L = r1 - r0, int(context_lens[s])
        if C == 0:
            continue
        if C > L:
            raise ValueError(f"sequence {s}: chunk of {C} rows longer than its context {L}")
        kb, vb = gather_seq(kc, vc, block_tables[s], L, bs=bs)
        K = dequant(kb, cache_dtype, k_scale)
        V = dequant(vb, cache_dtype, v_scale)
        G = H_q // K.shape[1]
        pos = L - C + np.arange(C)                        # position of each chunk row
        hidden = np.arange(L)[None, :] > pos[:, None]     # [C, L]: token after the row
        for g in range(H_q):
            h = g // G
            Z = sc * (q[r0:r1, g] @ K[:, h].T)
            Z[hidden] = -np.inf
            E = np.exp(Z - Z.max(axis=1, keepdims=True))
            W = E / E.sum(axis=1, keepdims=True)
            out[r0:r1, g] = W @ V[:, h]
    return out
