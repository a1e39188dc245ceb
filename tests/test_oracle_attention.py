"""Pins of the oracle's fp64 decode attention.

The oracle gathers through block tables and then applies the definition of
softmax attention; these tests pin it to things other than itself: torch's
scaled_dot_product_attention on the contiguous cache, closed forms,
hand-computed examples, and a pure-Python evaluation on tiny inputs.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import synth
from oracle import attention as A
from oracle import layout as Lx
from oracle import replay
from oracle.formats import decode


def _sdpa(q, Ks, Vs, scale):
    """torch SDPA in fp64 over contiguous per-sequence K/V; GQA via enable_gqa."""
    outs = []
    for s in range(q.shape[0]):
        qq = torch.from_numpy(q[s])[:, None, :][None]           # [1, H_q, 1, d]
        kk = torch.from_numpy(Ks[s]).permute(1, 0, 2)[None]     # [1, H_kv, L, d]
        vv = torch.from_numpy(Vs[s]).permute(1, 0, 2)[None]
        o = Fn.scaled_dot_product_attention(qq, kk.contiguous(), vv.contiguous(),
                                            scale=float(np.float32(scale)),
                                            enable_gqa=qq.shape[1] != kk.shape[1])
        outs.append(o[0, :, 0, :].numpy())
    return np.stack(outs)


def _torch_fp8_roundtrip(bf16_bits, scale):
    """bf16 rows -> E4M3FN by torch -> fp64 values, with a per-tensor scale:
    x * fp32(1 / scale) in fp32, clamped to the format's +-448 (torch's cast
    does not saturate), cast to float8_e4m3fn (round to nearest even), then
    widened and multiplied by the scale in fp64."""
    x = torch.from_numpy(np.ascontiguousarray(bf16_bits).view(np.int16)).view(torch.bfloat16)
    inv = torch.tensor(np.float32(1.0) / np.float32(scale), dtype=torch.float32)
    y = torch.clamp(x.float() * inv, -448.0, 448.0)
    return y.to(torch.float8_e4m3fn).to(torch.float64).numpy() * float(np.float32(scale))


def _pyloop(q, K, V, scale):
    """Tiny pure-Python decode attention, math.fsum accumulation."""
    L = len(K)
    z = [float(np.float32(scale)) * math.fsum(qi * ki for qi, ki in zip(q, K[t])) for t in range(L)]
    m = max(z)
    e = [math.exp(zt - m) for zt in z]
    tot = math.fsum(e)
    return [math.fsum(e[t] * V[t][i] for t in range(L)) / tot for i in range(len(V[0]))]


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_paged_oracle_matches_sdpa_on_contiguous_cache(cfg_id):
    wl = synth.make(synth.SMALL[cfg_id])
    c = wl.cfg
    st, _ = replay.build(wl)
    tables = st.tables(c.S)
    out, wsum = A.paged_decode(wl.q, c.q_dtype, st.kc, st.vc, tables, wl.context_lens,
                               bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale,
                               k_scale=c.k_scale, v_scale=c.v_scale)
    # contiguous cache straight from the value streams (never paged); fp8
    # values are quantised and dequantised by torch's float8_e4m3fn type with
    # each pool's own scale (keys and values have different scales in the
    # small skewed workload)
    Ks, Vs = [], []
    for s in range(c.S):
        parts = []
        if c.prefix:
            parts.append(wl.values(("prefix",), 0, c.prefix))
        own = int(wl.context_lens[s]) - c.prefix
        parts.append(wl.values(("seq", s), 0, own))
        kb = np.concatenate([p[0] for p in parts])
        vb = np.concatenate([p[1] for p in parts])
        if c.kv_dtype == "fp8":
            Ks.append(_torch_fp8_roundtrip(kb, c.k_scale))
            Vs.append(_torch_fp8_roundtrip(vb, c.v_scale))
        else:
            Ks.append(decode(kb, c.kv_dtype))
            Vs.append(decode(vb, c.kv_dtype))
    ref = _sdpa(decode(wl.q, c.q_dtype), Ks, Vs, c.scale)
    assert np.abs(out - ref).max() < 1e-12
    assert np.abs(wsum - 1.0).max() < 1e-12


def test_gqa_head_mapping_matches_sdpa():
    rng = np.random.default_rng(7)
    S, Hq, Hkv, d, L = 2, 8, 2, 16, 9
    q = rng.standard_normal((S, Hq, d))
    Ks = [rng.standard_normal((L, Hkv, d)) for _ in range(S)]
    Vs = [rng.standard_normal((L, Hkv, d)) for _ in range(S)]
    out, _ = A.dense_decode(q, Ks, Vs, 0.25)
    assert np.abs(out - _sdpa(q, Ks, Vs, 0.25)).max() < 1e-13
    # a plausible wrong mapping (g % H_kv) must disagree
    wrong = np.stack([[A.attend_one(q[s, g], Ks[s][:, g % Hkv], Vs[s][:, g % Hkv], 0.25)[0]
                       for g in range(Hq)] for s in range(S)])
    assert np.abs(out - wrong).max() > 1e-3


def test_golden_tiny_examples(golden_dir):
    with open(os.path.join(golden_dir, "attention_tiny.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        o, w = A.attend_one(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), c["scale"])
        assert np.abs(o - np.array(c["out"])).max() < 1e-15, c["name"]
        assert abs(w - 1.0) < 1e-15


def test_pure_python_bruteforce_on_tiny_paged_inputs():
    rng = np.random.default_rng(8)
    NB, H, d, bs = 12, 2, 8, 4
    kc, vc = Lx.empty_pools(NB, H, d, bs, "f32", fill=0)
    lens = [1, 3, 4, 9]
    order = rng.permutation(NB)
    tables, pos, rows = [], 0, []
    for L in lens:
        n = -(-L // bs)
        tables.append(order[pos:pos + n])
        pos += n
        k = rng.standard_normal((L, H, d)).astype(np.float32)
        v = rng.standard_normal((L, H, d)).astype(np.float32)
        t = np.arange(L)
        Lx.write_kv(kc, vc, k, v, tables[-1][t // bs] * bs + t % bs, bs=bs, src_dtype="f32",
                    cache_dtype="f32")
        rows.append((k, v))
    Hq = 4
    q = rng.standard_normal((len(lens), Hq, d)).astype(np.float32)
    tab = np.full((len(lens), 3), -1)
    for s, t in enumerate(tables):
        tab[s, :len(t)] = t
    out, _ = A.paged_decode(q, "f32", kc, vc, tab, lens, bs=bs, cache_dtype="f32", scale=0.3)
    for s, L in enumerate(lens):
        for g in range(Hq):
            h = g // (Hq // H)
            K = [[float(x) for x in rows[s][0][t, h]] for t in range(L)]
            V = [[float(x) for x in rows[s][1][t, h]] for t in range(L)]
            ref = _pyloop([float(x) for x in q[s, g]], K, V, 0.3)
            assert np.abs(out[s, g] - np.array(ref)).max() < 1e-13


def test_closed_forms():
    rng = np.random.default_rng(9)
    d = 32
    V = rng.standard_normal((10, d))
    K = rng.standard_normal((10, d))
    # L = 1 returns its value row exactly
    o, _ = A.attend_one(rng.standard_normal(d), K[:1], V[:1], 0.7)
    assert (o == V[0]).all()
    # q = 0 (or scale = 0) returns the mean of the rows
    o, _ = A.attend_one(np.zeros(d), K, V, 0.7)
    assert np.abs(o - V.mean(0)).max() < 1e-15
    o, _ = A.attend_one(rng.standard_normal(d), K, V, 0.0)
    assert np.abs(o - V.mean(0)).max() < 1e-15
    # constant value rows return the constant
    o, w = A.attend_one(rng.standard_normal(d), K, np.full((10, d), 2.5), 0.7)
    assert np.abs(o - 2.5).max() < 1e-14 and abs(w - 1) < 1e-15
    # one key aligned with q and much larger than the others picks its row
    q = rng.standard_normal(d)
    K2 = np.zeros((10, d))
    K2[6] = 30 * q / np.linalg.norm(q)
    o, _ = A.attend_one(q / np.linalg.norm(q), K2, V, 1.0)
    assert np.abs(o - V[6]).max() < 1e-10
    # two keys: logistic weights
    K3 = rng.standard_normal((2, d))
    qq = rng.standard_normal(d)
    z = 0.375 * (K3 @ qq)   # 0.375 is exact in fp32
    w0 = 1.0 / (1.0 + math.exp(-(z[0] - z[1])))
    o, _ = A.attend_one(qq, K3, V[:2], 0.375)
    assert np.abs(o - (w0 * V[0] + (1 - w0) * V[1])).max() < 1e-14


def test_empty_context_returns_zeros():
    o, w = A.attend_one(np.ones(8), np.zeros((0, 8)), np.zeros((0, 8)), 1.0)
    assert (o == 0).all() and w == 0.0


def test_prefix_shared_equals_private_copies():
    wl = synth.make(synth.SMALL[4])
    c = wl.cfg
    st, _ = replay.build(wl)
    # sharing really happened: full prefix blocks are referenced by every sequence
    shared = st.model.table(0)[: c.prefix // c.bs]
    assert all(st.model.refcount(b) == c.S for b in shared)
    assert len(st.cow_log) == c.S - 1
    out, _ = A.paged_decode(wl.q, c.q_dtype, st.kc, st.vc, st.tables(c.S), wl.context_lens,
                            bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale)
    wp = synth.private_copy(wl)
    st2, _ = replay.build(wp)
    out2, _ = A.paged_decode(wp.q, c.q_dtype, st2.kc, st2.vc, st2.tables(c.S), wp.context_lens,
                             bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale)
    assert (out == out2).all()


def test_block_order_does_not_change_the_result():
    wl = synth.make(synth.SMALL[3])
    c = wl.cfg
    st, _ = replay.build(wl)
    out, _ = A.paged_decode(wl.q, c.q_dtype, st.kc, st.vc, st.tables(c.S), wl.context_lens,
                            bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale)
    w2 = synth.with_free_order(wl, np.random.default_rng(99).permutation(wl.num_blocks))
    st2, _ = replay.build(w2)
    assert not np.array_equal(st.tables(c.S), st2.tables(c.S))
    out2, _ = A.paged_decode(w2.q, c.q_dtype, st2.kc, st2.vc, st2.tables(c.S), w2.context_lens,
                             bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale)
    assert (out == out2).all()
