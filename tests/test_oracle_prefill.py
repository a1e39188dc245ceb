"""Pins of the oracle's fp64 chunked prefill (causal attention of each
sequence's last C positions over its paged cache).

Each test pins ``oracle.attention.paged_prefill`` to something other than
itself: torch's scaled_dot_product_attention with an explicit causal mask on
the contiguous (never paged) cache, a pure-Python fsum evaluation on tiny
paged inputs, the running mean that q = 0 must give (an off-by-one in the
causal boundary changes it), the first position of a fresh prompt, and the
decode output for the last row of every chunk.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import synth
from oracle import attention as A
from oracle import layout as Lx
from oracle import replay
from oracle.formats import decode


def _workload(G=4, **kw):
    base = synth.PREFILL["small"]
    return synth.make(dataclasses.replace(base, H_q=base.H_kv * G, **kw))


def _contiguous(wl, s):
    """K, V fp64 [L, H_kv, d] of sequence s straight from its value stream."""
    c = wl.cfg
    kb, vb = wl.values(("seq", s), 0, int(wl.context_lens[s]))
    return decode(kb, c.kv_dtype), decode(vb, c.kv_dtype)


def _oracle(wl, st, chunks, q_bits, seqs=None):
    c = wl.cfg
    qs = np.concatenate([[0], np.cumsum(chunks)])
    return A.paged_prefill(q_bits, c.q_dtype, st.kc, st.vc, st.tables(c.S), wl.context_lens, qs,
                           bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale, seqs=seqs), qs


@pytest.mark.parametrize("G", [4, 1, 8])
def test_prefill_matches_sdpa_with_causal_mask(G):
    wl = _workload(G)
    c = wl.cfg
    st, _ = replay.build(wl)
    chunks = synth.prefill_chunks(wl)
    q_bits = synth.prefill_queries(wl, chunks)
    out, qs = _oracle(wl, st, chunks, q_bits)
    q = decode(q_bits, c.q_dtype)
    for s in range(c.S):
        L, C = int(wl.context_lens[s]), int(chunks[s])
        K, V = _contiguous(wl, s)
        qq = torch.from_numpy(q[qs[s]:qs[s + 1]]).permute(1, 0, 2)[None]   # [1, H_q, C, d]
        kk = torch.from_numpy(K).permute(1, 0, 2)[None].contiguous()       # [1, H_kv, L, d]
        vv = torch.from_numpy(V).permute(1, 0, 2)[None].contiguous()
        allowed = torch.arange(L)[None, :] <= (L - C + torch.arange(C))[:, None]
        ref = Fn.scaled_dot_product_attention(qq, kk, vv, attn_mask=allowed,
                                              scale=float(np.float32(c.scale)),
                                              enable_gqa=G != 1)
        ref = ref[0].permute(1, 0, 2).numpy()
        assert np.abs(out[qs[s]:qs[s + 1]] - ref).max() < 1e-12, s


def test_prefill_pure_python_on_tiny_paged_inputs():
    rng = np.random.default_rng(61)
    NB, H, d, bs, Hq = 16, 2, 8, 4, 4
    kc, vc = Lx.empty_pools(NB, H, d, bs, "f32", fill=0)
    lens, chunks = [5, 9, 3], [2, 9, 1]
    order = rng.permutation(NB)
    tables, pos, rows = np.full((3, 4), -1), 0, []
    for s, L in enumerate(lens):
        n = -(-L // bs)
        tables[s, :n] = order[pos:pos + n]
        pos += n
        k = rng.standard_normal((L, H, d)).astype(np.float32)
        v = rng.standard_normal((L, H, d)).astype(np.float32)
        t = np.arange(L)
        Lx.write_kv(kc, vc, k, v, tables[s][t // bs] * bs + t % bs, bs=bs, src_dtype="f32",
                    cache_dtype="f32")
        rows.append((k.astype(np.float64), v.astype(np.float64)))
    T = sum(chunks)
    q = rng.standard_normal((T, Hq, d)).astype(np.float32)
    qs = np.concatenate([[0], np.cumsum(chunks)])
    out = A.paged_prefill(q, "f32", kc, vc, tables, np.array(lens), qs, bs=bs, cache_dtype="f32",
                          scale=0.3)
    sc = float(np.float32(0.3))
    for s, (L, C) in enumerate(zip(lens, chunks)):
        K, V = rows[s]
        for i in range(C):
            p = L - C + i
            r = qs[s] + i
            for g in range(Hq):
                h = g // (Hq // H)
                z = [sc * math.fsum(float(q[r, g, j]) * K[t, h, j] for j in range(d))
                     for t in range(p + 1)]
                m = max(z)
                e = [math.exp(zt - m) for zt in z]
                tot = math.fsum(e)
                want = [math.fsum(e[t] * V[t, h, j] for t in range(p + 1)) / tot for j in range(d)]
                assert np.abs(out[r, g] - np.array(want)).max() < 1e-13


def test_prefill_zero_query_gives_running_mean():
    """q = 0 makes every visible token weigh the same: row i returns the mean
    of the value rows at positions 0 .. L - C + i."""
    wl = _workload(4)
    c = wl.cfg
    st, _ = replay.build(wl)
    chunks = synth.prefill_chunks(wl)
    q_bits = np.zeros((int(chunks.sum()), c.H_q, c.d), dtype=np.uint16)
    out, qs = _oracle(wl, st, chunks, q_bits)
    G = c.H_q // c.H_kv
    for s in range(c.S):
        L, C = int(wl.context_lens[s]), int(chunks[s])
        _, V = _contiguous(wl, s)
        run = np.cumsum(V, axis=0) / np.arange(1, L + 1)[:, None, None]   # mean of rows 0..t
        for i in range(C):
            want = run[L - C + i]                                            # [H_kv, d]
            got = out[qs[s] + i]
            assert np.abs(got - np.repeat(want, G, axis=0)).max() < 1e-13


def test_prefill_first_position_returns_first_value():
    """A chunk that is the whole context (a fresh prompt): its first row sees
    only token 0, so it returns that token's value row exactly."""
    wl = _workload(4)
    c = wl.cfg
    st, _ = replay.build(wl)
    chunks = wl.context_lens.copy()
    q_bits = synth.prefill_queries(wl, chunks)
    out, qs = _oracle(wl, st, chunks, q_bits)
    G = c.H_q // c.H_kv
    for s in range(c.S):
        _, V = _contiguous(wl, s)
        assert np.array_equal(out[qs[s]], np.repeat(V[0], G, axis=0))


def test_prefill_last_row_equals_decode():
    wl = _workload(4)
    c = wl.cfg
    st, _ = replay.build(wl)
    chunks = synth.prefill_chunks(wl)
    q_bits = synth.prefill_queries(wl, chunks)
    out, qs = _oracle(wl, st, chunks, q_bits)
    last = q_bits[qs[1:] - 1]                                  # [S, H_q, d]
    dec, _ = A.paged_decode(last, c.q_dtype, st.kc, st.vc, st.tables(c.S), wl.context_lens,
                            bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale)
    assert np.abs(out[qs[1:] - 1] - dec).max() < 1e-13


def test_prefill_rejects_chunk_longer_than_context():
    wl = _workload(4)
    c = wl.cfg
    st, _ = replay.build(wl)
    chunks = wl.context_lens.copy()
    chunks[1] += 1
    with pytest.raises(ValueError):
        _oracle(wl, st, chunks, synth.prefill_queries(wl, chunks))
