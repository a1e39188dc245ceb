"""Pins of the oracle's block layout, scatter and gather."""

import json
import os

import numpy as np
import pytest

from oracle import layout as Lx
from oracle.formats import STORAGE


def _bits(rng, shape, dtype):
    if dtype == "f32":
        return rng.standard_normal(shape).astype(np.float32)
    if dtype == "bf16":
        return rng.integers(0, 0x7F00, size=shape, dtype=np.uint16)
    return rng.integers(0, 0x7F, size=shape, dtype=np.uint8)


def test_layout_offsets_golden(golden_dir):
    with open(os.path.join(golden_dir, "layout_offsets.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        kw = dict(H_kv=c["H_kv"], d=c["d"], bs=c["bs"])
        assert Lx.key_offset(c["b"], c["h"], c["o"], c["i"], dtype=c["dtype"], **kw) == c["key"]
        assert Lx.value_offset(c["b"], c["h"], c["o"], c["i"], **kw) == c["value"]
        # and write_kv really stores the element there
        kc, vc = Lx.empty_pools(c["nb"], c["H_kv"], c["d"], c["bs"], c["dtype"])
        T = 1
        k = np.zeros((T, c["H_kv"], c["d"]), dtype=STORAGE[c["dtype"]])
        v = np.zeros_like(k)
        k[0, c["h"], c["i"]] = 7
        v[0, c["h"], c["i"]] = 9
        Lx.write_kv(kc, vc, k, v, [c["b"] * c["bs"] + c["o"]], bs=c["bs"],
                    src_dtype=c["dtype"], cache_dtype=c["dtype"])
        kf, vf = kc.reshape(-1), vc.reshape(-1)
        assert kf[c["key"]] == 7 and np.count_nonzero(kf) == 1
        assert vf[c["value"]] == 9 and np.count_nonzero(vf) == 1


@pytest.mark.parametrize("dtype,d,bs", [("f32", 64, 16), ("bf16", 128, 16), ("fp8", 128, 32), ("bf16", 64, 32)])
def test_write_then_gather_roundtrip(dtype, d, bs):
    rng = np.random.default_rng(2)
    H, NB = 3, 20
    lens = [1, bs, bs + 1, 3 * bs - 1]
    order = rng.permutation(NB)
    tables, pos = [], 0
    for L in lens:
        nblk = -(-L // bs)
        tables.append(order[pos:pos + nblk])
        pos += nblk
    kc, vc = Lx.empty_pools(NB, H, d, bs, dtype, fill=0)
    rows = []
    for s, L in enumerate(lens):
        k = _bits(rng, (L, H, d), dtype)
        v = _bits(rng, (L, H, d), dtype)
        t = np.arange(L)
        slots = tables[s][t // bs] * bs + t % bs
        Lx.write_kv(kc, vc, k, v, slots, bs=bs, src_dtype=dtype, cache_dtype=dtype)
        rows.append((k, v))
    for s, L in enumerate(lens):
        gk, gv = Lx.gather_seq(kc, vc, tables[s], L, bs=bs)
        assert gk.tobytes() == rows[s][0].tobytes()
        assert gv.tobytes() == rows[s][1].tobytes()


def test_negative_slots_are_skipped():
    kc, vc = Lx.empty_pools(4, 2, 64, 16, "f32", fill=0)
    k = np.ones((3, 2, 64), np.float32)
    Lx.write_kv(kc, vc, k, k, [-1, 5, -7], bs=16, src_dtype="f32", cache_dtype="f32")
    assert np.count_nonzero(kc) == 2 * 64 and np.count_nonzero(vc) == 2 * 64


def test_permuting_physical_blocks_keeps_every_gather():
    rng = np.random.default_rng(3)
    NB, H, d, bs = 16, 2, 128, 16
    kc = _bits(rng, (NB, H, d // 8, bs, 8), "bf16")
    vc = _bits(rng, (NB, H, d, bs), "bf16")
    table = rng.permutation(NB)[:5]
    L = 5 * bs - 3
    ref = Lx.gather_seq(kc, vc, table, L, bs=bs)
    pi = rng.permutation(NB)            # physical block b moves to pi[b]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi], vc2[pi] = kc, vc
    got = Lx.gather_seq(kc2, vc2, pi[table], L, bs=bs)
    assert got[0].tobytes() == ref[0].tobytes() and got[1].tobytes() == ref[1].tobytes()


def test_copy_blocks():
    rng = np.random.default_rng(4)
    kc = _bits(rng, (6, 2, 8, 16, 8), "bf16")
    vc = _bits(rng, (6, 2, 64, 16), "bf16")
    k0, v0 = kc.copy(), vc.copy()
    Lx.copy_blocks(kc, vc, [(1, 4), (2, 5)])
    assert (kc[4] == k0[1]).all() and (vc[5] == v0[2]).all()
    assert (kc[:4] == k0[:4]).all()


def test_fp8_write_quantises():
    from oracle.formats import quantize_fp8
    rng = np.random.default_rng(5)
    kc, vc = Lx.empty_pools(2, 1, 128, 32, "fp8", fill=0)
    bits = rng.integers(0, 0x4400, size=(1, 1, 128), dtype=np.uint16)
    Lx.write_kv(kc, vc, bits, bits, [33], bs=32, src_dtype="bf16", cache_dtype="fp8",
                k_scale=0.05, v_scale=0.5)
    gk, gv = Lx.gather_seq(kc, vc, [0, 1], 34, bs=32)
    assert (gk[33] == quantize_fp8(bits[0], "bf16", 0.05)).all()
    assert (gv[33] == quantize_fp8(bits[0], "bf16", 0.5)).all()


def test_move_blocks_between_pools():
    """move_blocks (swapping sequences between a device pool and a host pool)
    on pools where every byte of block b in pool p holds a known value: the
    listed destination blocks take their sources' bytes, every other block
    keeps its own, the source pool is unchanged, and moving back with the
    pairs reversed restores the original destination contents."""
    H, d, bs = 2, 64, 16
    dev_k, dev_v = Lx.empty_pools(5, H, d, bs, "bf16", fill=0)
    host_k, host_v = Lx.empty_pools(4, H, d, bs, "bf16", fill=0)
    for b in range(5):
        dev_k[b], dev_v[b] = 0x1000 + b, 0x2000 + b
    for b in range(4):
        host_k[b], host_v[b] = 0x3000 + b, 0x4000 + b
    d0 = (dev_k.copy(), dev_v.copy())
    h0 = (host_k.copy(), host_v.copy())
    pairs = [(3, 0), (0, 2), (4, 1)]           # (device block, host slot)
    Lx.move_blocks(host_k, host_v, dev_k, dev_v, pairs)
    assert [int(host_k[h].flat[0]) for h in range(4)] == [0x1003, 0x1004, 0x1000, 0x3003]
    assert [int(host_v[h].flat[0]) for h in range(4)] == [0x2003, 0x2004, 0x2000, 0x4003]
    for h in range(4):                         # whole blocks move, not just their first element
        assert (host_k[h] == host_k[h].flat[0]).all() and (host_v[h] == host_v[h].flat[0]).all()
    assert (dev_k == d0[0]).all() and (dev_v == d0[1]).all()
    # into a fresh device pool and back out: the round trip restores the host pool
    new_k, new_v = Lx.empty_pools(5, H, d, bs, "bf16", fill=0)
    Lx.move_blocks(new_k, new_v, host_k, host_v, [(h, b) for b, h in pairs])
    assert [int(new_k[b].flat[0]) for b in range(5)] == [0x1000, 0, 0, 0x1003, 0x1004]
    host_k[...], host_v[...] = h0
    Lx.move_blocks(host_k, host_v, new_k, new_v, pairs)
    Lx.move_blocks(host_k, host_v, *h0, [(3, 3)])
    assert [int(host_k[h].flat[0]) for h in range(4)] == [0x1003, 0x1004, 0x1000, 0x3003]
