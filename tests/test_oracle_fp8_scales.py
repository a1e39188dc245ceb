"""Pins of the oracle's fp8 per-tensor scales: the key scale multiplies the
keys and only the keys, the value scale the values and only the values, on
the way in (quantise on write) and on the way out (dequantise before
attention).  The skewed long-context workload stores its cache as fp8 with a
per-tensor scale; the pages ask for narrow storage with fp32 accumulation
("PagedAttention Kernel：大模型推理优化的显存管理革新" §6).

Expected values here are closed forms worked out by hand from the E4M3FN
format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits) and from the
logistic form of a two-token softmax, not from the oracle's own code.
"""

import math

import numpy as np

import synth
from oracle import attention as OA
from oracle import layout as OL
from oracle import replay

# E4M3FN codes: 0.5 = 2^-1 (exponent field 6), 1.0 (7), 2.0 (8), 4.0 (9)
E4M3 = {0.5: 0x30, 1.0: 0x38, 2.0: 0x40, 4.0: 0x48}
BF16_ONE = 0x3F80


def _two_token_cache():
    """One sequence of two tokens in block 1 of a two-block fp8 pool, one kv
    head, head_dim 16, block size 16: key dim 0 holds codes 1.0 and 2.0, value
    dim 0 holds codes 1.0 and 4.0, every other element is code 0 (+0.0)."""
    kc, vc = OL.empty_pools(2, 1, 16, 16, "fp8", fill=0)
    # key [block, head, dim // 16, slot, dim % 16]; value [block, head, dim, slot]
    kc[1, 0, 0, 0, 0] = E4M3[1.0]
    kc[1, 0, 0, 1, 0] = E4M3[2.0]
    vc[1, 0, 0, 0] = E4M3[1.0]
    vc[1, 0, 0, 1] = E4M3[4.0]
    return kc, vc


def test_dequant_routes_key_and_value_scales():
    kc, vc = _two_token_cache()
    q = np.zeros((1, 1, 16), np.uint16)
    q[0, 0, 0] = BF16_ONE
    out, wsum = OA.paged_decode(q, "bf16", kc, vc, np.array([[1]]), [2], bs=16, cache_dtype="fp8",
                                scale=0.5, k_scale=0.25, v_scale=2.0)
    # scores 0.5 * 0.25 * {1, 2}; weight of token 1 = logistic(0.25 - 0.125)
    w1 = 1.0 / (1.0 + math.exp(-0.125))
    want0 = 2.0 * ((1.0 - w1) * 1.0 + w1 * 4.0)
    assert abs(out[0, 0, 0] - want0) < 1e-15
    assert (out[0, 0, 1:] == 0).all() and abs(wsum[0, 0] - 1) < 1e-15
    # the same cache with the two scales exchanged gives another value
    sw, _ = OA.paged_decode(q, "bf16", kc, vc, np.array([[1]]), [2], bs=16, cache_dtype="fp8",
                            scale=0.5, k_scale=2.0, v_scale=0.25)
    w1s = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(sw[0, 0, 0] - 0.25 * (1.0 + 3.0 * w1s)) < 1e-15
    assert abs(sw[0, 0, 0] - want0) > 1.0


def test_write_routes_key_and_value_scales():
    kc, vc = OL.empty_pools(2, 1, 16, 16, "fp8", fill=0)
    k = np.zeros((1, 1, 16), np.uint16)
    v = np.zeros((1, 1, 16), np.uint16)
    k[0, 0, 0] = BF16_ONE
    v[0, 0, 0] = BF16_ONE
    OL.write_kv(kc, vc, k, v, [16 + 3], bs=16, src_dtype="bf16", cache_dtype="fp8",
                k_scale=0.25, v_scale=2.0)
    # key 1.0 / 0.25 = 4.0, value 1.0 / 2.0 = 0.5, both exact in E4M3FN
    assert kc[1, 0, 0, 3, 0] == E4M3[4.0]
    assert vc[1, 0, 0, 3] == E4M3[0.5]
    assert np.count_nonzero(kc) == 1 and np.count_nonzero(vc) == 1


def test_small_skewed_workload_is_sensitive_to_a_scale_swap():
    """The small fp8 workload the GPU parity tests run has distinct key and
    value scales; an oracle with the two scales exchanged (a mistake planted
    here, on the CPU) disagrees with the correct one far beyond the fp8
    tolerance, on the write and on the attention, so a kernel that exchanged
    them could not pass those tests."""
    wl = synth.make(synth.SMALL[5])
    c = wl.cfg
    assert c.kv_dtype == "fp8" and c.k_scale != c.v_scale
    st, _ = replay.build(wl)
    ref, _ = OA.paged_decode(wl.q, c.q_dtype, st.kc, st.vc, st.tables(c.S), wl.context_lens,
                             bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale, k_scale=c.k_scale,
                             v_scale=c.v_scale)
    bad, _ = OA.paged_decode(wl.q, c.q_dtype, st.kc, st.vc, st.tables(c.S), wl.context_lens,
                             bs=c.bs, cache_dtype=c.kv_dtype, scale=c.scale, k_scale=c.v_scale,
                             v_scale=c.k_scale)
    assert np.abs(bad - ref).max() > 10 * 6e-2
    # write side: the codes of one sequence's rows stored with the scales exchanged
    k, v = wl.values(("seq", 0), 0, 64)
    good_k = OL.encode_for_cache(k, c.src_dtype, "fp8", c.k_scale)
    swap_k = OL.encode_for_cache(k, c.src_dtype, "fp8", c.v_scale)
    assert np.mean(good_k != swap_k) > 0.5
