"""8-bit floating-point KV storage (OCP E4M3).  (Test infrastructure.)

Source: "LLM推理优化：技术原理解析总览" (dpshk.com), §5.1: keeping the KV cache
in 16-bit precision wastes memory next to a quantised model; the remedy given
is an FP8 KV cache. The page names neither the 8-bit format nor how values
are scaled. Readings:

* the format is OCP E4M3 ("FN"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds subnormals m/8 · 2^-6; the codes
  0x7F and 0xFF are NaN; there is no infinity; the largest finite magnitude
  is 448 (code 0x7E);
* one scale per pool for K and one for V (per-tensor): the stored value is
  x / scale, and a stored code c stands for decode(c) · scale;
* quantisation: x (bf16, exact in fp32) is divided by the scale in fp32 with
  IEEE round-to-nearest-even (the result is the fp32 number nearest the exact
  quotient), clamped to [-448, 448], then rounded to the nearest E4M3 value,
  ties to the code with an even mantissa (its lowest bit 0).

This module holds the format's definition only: the 256-entry value table
built from the bit fields, and nearest-value rounding over that table.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_value", "e4m3_table", "decode_e4m3", "quantize_e4m3", "NAN_CODE"]

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code from its bit fields (NaN for 0x7F / 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """fp64 values of all 256 codes (a copy)."""
    return _TABLE.copy()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> fp64 values (exact)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


# Non-negative finite codes 0x00..0x7E in increasing value order.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALS = _TABLE[:0x7F]


def quantize_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    """fp32-representable values -> uint8 E4M3 codes of x / scale.

    The quotient is taken in fp32 (NumPy's fp32 division is IEEE
    round-to-nearest-even), clamped to ±448, then rounded to the nearest
    finite E4M3 value; a tie goes to the code with an even mantissa. The sign
    is kept separately, so -0.0 and tiny negatives give code 0x80. A NaN
    quotient gives the NaN code 0x7F with the input's sign bit.
    """
    x = np.asarray(x, dtype=np.float32)
    q = (x / np.float32(scale)).astype(np.float32)
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float64)
    mag = np.abs(q)
    # index of the largest table value <= mag, and the next one up
    lo = np.searchsorted(_POS_VALS, mag, side="right") - 1
    lo = np.clip(lo, 0, len(_POS_VALS) - 1)
    hi = np.minimum(lo + 1, len(_POS_VALS) - 1)
    d_lo = mag - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.isnan(q), np.uint8(NAN_CODE), code).astype(np.uint8)
    neg = np.signbit(q)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
