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
  e2m1  : OCP FP4 E2M1: 2 significant bits, exponent bias 1, normal range from 1,
          subnormal spacing 0.5, largest finite 6, no infinities or NaN.
          Saturating conversion: magnitudes beyond 6 become 6.
  mxfp4 : OCP microscaling (MX) blocks of 32 consecutive e2m1 elements sharing
          one E8M0 scale 2**X, X in [-127, 127], stored as the byte X + 127.  The
          pages say only that the lightning indexer uses FP4; MXFP4 is the FP4
          block format with a shared scale that the gfx950 matrix cores and
          conversion instructions define, so it is the reading taken here.
          X = floor(log2(max |v|)) - 2 (2 being the exponent of e2m1's largest
          power of two), clamped to [-127, 127]; an all-zero block takes
          X = -127.  Elements are the saturating RNE e2m1 conversion of v / 2**X.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
MX_BLOCK = 32


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


def round_e2m1(x) -> np.ndarray:
    """Saturating RNE conversion to e2m1 values."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E2M1_MAX, E2M1_MAX)
    return _round_nearest_even(x, 2, 0)


def e2m1_encode(r) -> np.ndarray:
    """4-bit codes (uint8 0..15) of e2m1 values r (r must already be representable):
    sign in bit 3, exponent field in bits 2..1, mantissa in bit 0."""
    r = np.asarray(r, dtype=np.float64)
    sign = np.signbit(r).astype(np.int64)
    a = np.abs(r)
    _, e = np.frexp(a)                      # a in [2**(e-1), 2**e)
    normal = a >= 1.0
    exp_field = np.where(normal, e - 1 + 1, 0)
    man = np.where(normal, a / np.ldexp(1.0, e - 1) - 1.0, a / 0.5) * np.where(normal, 2.0, 1.0)
    return ((sign << 3) | (exp_field.astype(np.int64) << 1) | man.astype(np.int64)).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    s = np.where((c >> 3) & 1, -1.0, 1.0)
    ef = (c >> 1) & 3
    mf = c & 1
    return s * np.where(ef > 0, (1.0 + mf / 2.0) * np.ldexp(1.0, ef - 1), mf * 0.5)


def mxfp4_quantize(c):
    """MXFP4 blocks of the rows of c [n][D] (D a multiple of 32).

    Returns (values fp64 [n][D] = element * 2**X, codes uint8 [n][D] (e2m1 codes),
    scale uint8 [n][D/32] (X + 127))."""
    c = np.asarray(c, dtype=np.float64)
    n, D = c.shape
    blk = c.reshape(n, D // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blk).max(axis=2)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))   # amax in [2**(e-1), 2**e): floor(log2 amax) = e - 1
    X = np.where(amax > 0, e - 1 - 2, -127)
    X = np.clip(X, -127, 127)
    r = round_e2m1(blk / np.ldexp(1.0, X)[:, :, None])
    values = (r * np.ldexp(1.0, X)[:, :, None]).reshape(n, D)
    return values, e2m1_encode(r).reshape(n, D), (X + 127).astype(np.uint8)


def mxfp4_dequantize(codes, scale) -> np.ndarray:
    """Values of MXFP4 codes [n][D] with scale bytes [n][D/32]."""
    codes = np.asarray(codes)
    n, D = codes.shape
    X = np.asarray(scale, dtype=np.int64) - 127
    v = e2m1_decode(codes).reshape(n, D // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, X)[:, :, None]
    return v.reshape(n, D)
