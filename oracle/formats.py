"""Element formats for the oracle (test infrastructure only).

Cache and query elements are stored as raw bits in numpy arrays:

  * ``"f32"``  -- numpy float32
  * ``"bf16"`` -- numpy uint16 holding the bfloat16 bit pattern
  * ``"fp8"``  -- numpy uint8 holding an OCP FP8 E4M3FN code

The pages fix only that attention accumulates in fp32 while storage may be
narrower ("PagedAttention Kernel：大模型推理优化的显存管理革新" §6, mixed
precision); the fp8 E4M3FN storage format and its per-tensor scale are a
reading of the workload, not of the pages.  Decoding is exact in fp64 for all
three formats.

Pins (tests/test_oracle_formats.py): the 256-code fp8 table against torch's
float8_e4m3fn and hand-written format constants (tests/golden/fp8_e4m3fn.json);
encode against torch's cast on in-range values, on every representable value
and on every midpoint between neighbours (ties to the even code), and on the
saturation and subnormal edge cases.
"""

from __future__ import annotations

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}

FP8_MAX = 448.0
FP8_NAN_CODE = 0x7F


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact fp64 (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _fp8_value(code: int) -> float:
    """Value of one E4M3FN code from the format's definition.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0
    holds subnormals m/8 * 2^-6; the pattern S.1111.111 is NaN; there are no
    infinities, so S.1111.110 = 1.75 * 2^8 = 448 is the largest finite value.
    """
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


FP8_TABLE = np.array([_fp8_value(c) for c in range(256)], dtype=np.float64)


def decode_fp8(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes -> exact fp64 values via the 256-entry table."""
    return FP8_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw stored bits of ``dtype`` -> exact fp64."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(bits)
    if dtype == "fp8":
        return decode_fp8(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


# Non-negative finite codes 0x00..0x7E in increasing value order (the code
# order is already monotone for this format).
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = FP8_TABLE[:0x7F]


def encode_fp8_from_f32(y: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3FN codes, round to nearest, ties to even, saturating.

    Written as the definition of rounding: pick the representable magnitude
    nearest to |y|; on an exact tie pick the one whose code is even (the code's
    low bit is the mantissa's low bit); magnitudes at or above the largest
    finite value 448 saturate to 448; NaN maps to the NaN code 0x7F.  The
    decision is taken on the fp32 value, compared exactly in fp64.
    """
    y = np.asarray(y, dtype=np.float32)
    flat = y.reshape(-1)
    mag = np.abs(flat.astype(np.float64))
    neg = np.signbit(flat)
    nan = np.isnan(flat)
    mag = np.where(nan, 0.0, mag)

    # index of the first representable value >= mag
    hi = np.searchsorted(_POS_VALUES, mag, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(mag >= FP8_MAX, 0x7E, code)
    code = np.where(neg, code | 0x80, code)  # sign bit kept, -0 -> 0x80
    code = np.where(nan, FP8_NAN_CODE, code)
    return code.astype(np.uint8).reshape(y.shape)


def f32_mul(a: np.ndarray, b) -> np.ndarray:
    """One correctly rounded fp32 multiply (numpy float32 arithmetic is IEEE)."""
    return (np.asarray(a, dtype=np.float32) * np.float32(b)).astype(np.float32)


def f32_reciprocal(s: float) -> np.float32:
    """fp32(1) / fp32(s), correctly rounded: the quantisation multiplier."""
    return np.float32(np.float32(1.0) / np.float32(s))


def quantize_fp8(x_bits: np.ndarray, src_dtype: str, scale: float) -> np.ndarray:
    """Quantise-on-write: stored code = E4M3FN(fp32(x) * fp32(1/scale)).

    ``scale`` is the dequantisation multiplier (value = decode(code) * scale);
    its fp32 reciprocal is formed once, then each element takes one fp32
    multiply and one saturating round-to-nearest-even into E4M3FN.
    """
    x32 = decode(x_bits, src_dtype).astype(np.float32)  # exact: f32/bf16 -> f32
    return encode_fp8_from_f32(f32_mul(x32, f32_reciprocal(scale)))
