"""Storage roundings used by the oracle, written from the number formats' definitions.

TEST INFRASTRUCTURE ONLY (see the package header).

All functions take and return float64 arrays holding exactly representable
values of the target format; rounding is to nearest, ties to even, done exactly
in float64 (scaling by powers of two and numpy.rint are exact).

Formats (the pages name fp8 storage for most KV entries and bf16 for part of
the KV: knightli.com DeepSeek-V4 KV-cache article, section "FP8 y FP4 reducen
aun mas el costo de cache"):
  bf16  : 8 significant bits, normal range from 2**-126, overflow to +-inf.
  e4m3  : OCP FP8 E4M3 "fn" variant: 4 significant bits, exponent bias 7,
          normal range from 2**-6, subnormal spacing 2**-9, largest finite 448,
          no infinities (the all-ones pattern is NaN).  Saturating conversion:
          magnitudes beyond 448 become 448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _round_nearest_even(x: np.ndarray, sig_bits: int, min_normal_exp: int) -> np.ndarray:
    """Round x to a binary format with `sig_bits` significant bits whose smallest
    normal is 2**min_normal_exp (gradual underflow below it)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # |x| in [2**(e-1), 2**e)
    e = np.maximum(e, min_normal_exp + 1)   # subnormals share the spacing of the lowest binade
    ulp = np.ldexp(1.0, e - sig_bits)
    return np.rint(x / ulp) * ulp


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    r = _round_nearest_even(x, 8, -126)
    big = np.ldexp(2.0 - 2.0 ** -7, 127)
    return np.where(np.abs(r) > big, np.copysign(np.inf, r), r)


def round_e4m3(x) -> np.ndarray:
    """Saturating RNE conversion to e4m3 values."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    return _round_nearest_even(x, 4, -6)


def e4m3_encode(r) -> np.ndarray:
    """Bit patterns (uint8) of e4m3 values r (r must already be representable)."""
    r = np.asarray(r, dtype=np.float64)
    sign = np.signbit(r).astype(np.uint8)
    a = np.abs(r)
    _, e = np.frexp(a)                      # a in [2**(e-1), 2**e)
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e - 1 + 7, 0)
    man = np.where(normal, a / np.ldexp(1.0, e - 1) - 1.0, a / 2.0 ** -9) * np.where(normal, 8.0, 1.0)
    code = (sign.astype(np.int64) << 7) | (exp_field.astype(np.int64) << 3) | man.astype(np.int64)
    return code.astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    ef = (c >> 3) & 15
    mf = c & 7
    val = np.where(ef > 0, (1.0 + mf / 8.0) * np.ldexp(1.0, ef - 7), mf * 2.0 ** -9)
    val = np.where((ef == 15) & (mf == 7), np.nan, val)
    return s * val


def bf16_bits(r) -> np.ndarray:
    """uint16 bit patterns of bf16 values r (exact: the upper half of their fp32 bits)."""
    f = np.asarray(r, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)
