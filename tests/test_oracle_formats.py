"""Pins of the oracle's element formats against the format definition and torch."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F


def _load(golden_dir):
    with open(os.path.join(golden_dir, "fp8_e4m3fn.json")) as f:
        return json.load(f)


def _num(v):
    return float(v) if not isinstance(v, str) else float(v)


def test_fp8_decode_golden(golden_dir):
    g = _load(golden_dir)
    for code_s, val in g["decode"].items():
        got = F.FP8_TABLE[int(code_s, 16)]
        want = _num(val)
        if math.isnan(want):
            assert math.isnan(got), code_s
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code_s


def test_fp8_decode_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.FP8_TABLE
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    # exactly two NaN codes, no infinities
    assert nan.sum() == 2 and not np.isinf(got).any()


def test_fp8_encode_golden(golden_dir):
    g = _load(golden_dir)
    xs = np.array([_num(a) for a, _ in g["encode"]], dtype=np.float32)
    want = np.array([int(c, 16) for _, c in g["encode"]], dtype=np.uint8)
    got = F.encode_fp8_from_f32(xs)
    assert (got == want).all(), list(zip(xs, got, want))


def test_fp8_encode_roundtrips_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = F.FP8_TABLE[codes].astype(np.float32)
    assert (F.encode_fp8_from_f32(vals) == codes).all()


def test_fp8_encode_midpoints_tie_to_even():
    pos = F.FP8_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert (mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2).all()  # exact in fp32
    got = F.encode_fp8_from_f32(mids).astype(np.int64)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert (got == want).all()
    assert (F.encode_fp8_from_f32(-mids).astype(np.int64) == (want | 0x80)).all()


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 50,
        rng.uniform(-447, 447, 100_000).astype(np.float32),
        (rng.standard_normal(100_000) * 1e-3).astype(np.float32),
    ])
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (F.encode_fp8_from_f32(x) == ref).all()


def test_quantize_is_one_fp32_multiply_then_round():
    # 3 * fp32(1/3) is not exactly 1 in fp32; the stored code must follow the
    # fp32 product, not the real quotient.
    scale = 3.0
    inv = F.f32_reciprocal(scale)
    assert inv == np.float32(1.0) / np.float32(3.0)
    x = np.array([3.0, 300.0, -1.5, 1e4], dtype=np.float32)
    codes = F.quantize_fp8(x, "f32", scale)
    want = F.encode_fp8_from_f32(np.float32(x) * inv)
    assert (codes == want).all()
    assert codes[3] == 0x7E  # 3333 saturates


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=100_000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = F.decode_bf16(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
