"""Pins of the oracle's storage roundings: exhaustive code tables, hand-derived
cases and torch's CPU casts (a library routine) where those are defined."""
import numpy as np
import pytest
import torch

from oracle import codecs


def test_e4m3_code_table_roundtrip():
    codes = np.arange(256)
    vals = codecs.e4m3_decode(codes)
    nan = np.isnan(vals)
    assert set(codes[nan]) == {0x7F, 0xFF}
    finite = codes[~nan]
    assert len(finite) == 254
    # every finite value is a fixed point of the rounding and encodes back to its code
    r = codecs.round_e4m3(vals[~nan])
    assert np.array_equal(r, vals[~nan])
    assert np.array_equal(codecs.e4m3_encode(r), finite.astype(np.uint8))
    assert np.max(vals[~nan]) == 448.0 and np.min(vals[~nan]) == -448.0
    pos = np.sort(vals[~nan][vals[~nan] > 0])
    assert pos[0] == 2.0 ** -9 and 2.0 ** -6 in pos
    # all e4m3 values are exact in bf16 (so dequantising to bf16 is lossless)
    assert np.array_equal(codecs.round_bf16(vals[~nan]), vals[~nan])


def test_e4m3_midpoints_tie_to_even():
    v = codecs.e4m3_decode(np.arange(128))          # non-negative codes 0..127
    ok = ~np.isnan(v)
    vals, codes = v[ok], np.arange(128)[ok]          # ascending with the code
    assert np.all(np.diff(vals) > 0)
    mids = (vals[:-1] + vals[1:]) / 2
    for sign in (1.0, -1.0):
        got = codecs.e4m3_encode(codecs.round_e4m3(sign * mids)).astype(np.int64) & 0x7F
        # the result is one of the two neighbours, the one whose mantissa field is even
        assert np.all((got == codes[:-1]) | (got == codes[1:]))
        assert np.all((got & 1) == 0)


def test_e4m3_matches_torch_cast_inside_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.normal(0, 0.01, 5000)]).astype(np.float32)
    vals = codecs.e4m3_decode(np.arange(256))
    vals = vals[~np.isnan(vals)]
    s = np.sort(np.unique(vals))
    mids = ((s[:-1] + s[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, s.astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.round_e4m3(x.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_e4m3_saturates():
    assert codecs.round_e4m3(np.array([1e6, -1e6, 460.0, 449.0])).tolist() == [448, -448, 448, 448]


def test_bf16_all_patterns_roundtrip():
    bits = np.arange(65536, dtype=np.uint32) << 16
    with np.errstate(invalid="ignore"):
        f = bits.view(np.float32).astype(np.float64)
    fin = np.isfinite(f)
    assert np.array_equal(codecs.round_bf16(f[fin]), f[fin])
    assert np.array_equal(codecs.bf16_bits(f[fin]), (bits[fin] >> 16).astype(np.uint16))


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, 1e-30, 1000),
                        rng.normal(0, 1e30, 1000)]).astype(np.float32)
    # exact midpoints: low 16 bits = 0x8000
    mids = ((rng.integers(0, 2 ** 15, 5000, dtype=np.uint32) << 17) | 0x8000).astype(np.uint32)
    mids = mids.view(np.float32)
    x = np.concatenate([x, mids[np.isfinite(mids)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(codecs.round_bf16(x.astype(np.float64)), ref)


def test_golden_e4m3_and_bf16(golden):
    for c in golden["e4m3"]["cases"]:
        r = codecs.round_e4m3(np.array([c["x"]]))
        assert r[0] == c["value"], c
        assert int(codecs.e4m3_encode(r)[0]) == c["code"], c
    for c in golden["bf16"]["cases"]:
        assert codecs.round_bf16(np.array([c["x"]]))[0] == c["value"], c


@pytest.mark.parametrize("fn", [codecs.round_bf16, codecs.round_e4m3, codecs.round_f32])
def test_rounding_idempotent_and_monotone(fn):
    rng = np.random.default_rng(2)
    x = np.sort(rng.normal(0, 4, 10000))
    r = fn(x)
    assert np.array_equal(fn(r), r)
    assert np.all(np.diff(r) >= 0)


# ---------------------------------------------------------------- FP4 (e2m1) and MXFP4 blocks
# OCP FP4 E2M1 value table (OCP Microscaling Formats specification, FP4 element
# format): the non-negative values 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7,
# the same negated for codes 8..15.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_code_table():
    vals = codecs.e2m1_decode(np.arange(16))
    assert np.array_equal(vals[:8], E2M1_TABLE)
    assert np.array_equal(vals[8:], [-v for v in E2M1_TABLE])
    assert np.signbit(vals[8]) and not np.signbit(vals[0])
    # fixed points of the rounding, encoding back to their codes; exact in bf16
    assert np.array_equal(codecs.round_e2m1(vals), vals)
    assert np.array_equal(codecs.e2m1_encode(vals), np.arange(16, dtype=np.uint8))
    assert np.array_equal(codecs.round_bf16(vals), vals)


def _nearest_e2m1_brute(x):
    """Nearest e2m1 value by exhaustive search over the table; ties to the code with
    an even mantissa bit; beyond +-6 the largest magnitude."""
    vals = np.array(E2M1_TABLE)
    out = np.empty_like(x)
    for i, v in enumerate(x):
        a = min(abs(v), 6.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            best = [b for b in best if b % 2 == 0]
        out[i] = np.copysign(vals[best[0]], v)
    return out


def test_e2m1_rounding_brute_force():
    grid = np.linspace(-8.0, 8.0, 16 * 64 + 1)                    # steps of 1/64: every midpoint is on it
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    x = np.concatenate([grid, mids, -mids, mids + 1e-9, mids - 1e-9, [7.0, 100.0, -1e30, 1e-40]])
    assert np.array_equal(codecs.round_e2m1(x), _nearest_e2m1_brute(x))


def test_mxfp4_hand_example():
    # 31 elements of 0.3 and one 5.0: max |v| = 5 lies in [4, 8), so floor(log2) = 2 and
    # X = 2 - 2 = 0 (scale byte 127); 0.3 rounds to 0.5 (above the 0.25 midpoint) and
    # 5.0 is the midpoint of 4 and 6, which goes to 4 (even mantissa bit).
    v, c, s = codecs.mxfp4_quantize(np.array([[0.3] * 31 + [5.0]]))
    assert s.tolist() == [[127]]
    assert np.array_equal(v[0], [0.5] * 31 + [4.0])
    assert c[0, 0] == 1 and c[0, 31] == 6


def _scale_exp_brute(amax):
    """Largest integer k with 2**k <= amax, by stepping (amax > 0)."""
    k = 0
    while 2.0 ** k > amax:
        k -= 1
    while 2.0 ** (k + 1) <= amax:
        k += 1
    return k


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mxfp4_blocks_brute_force(seed):
    rng = np.random.default_rng(seed)
    n, D = 24, 128
    c = rng.standard_normal((n, D)) * np.ldexp(1.0, rng.integers(-30, 30, size=(n, 1)))
    c[0] = 0.0                                      # an all-zero row: four zero blocks
    c[1, :32] = 0.0
    c[1, 5] = -3.0                                  # a single nonzero element
    c[2, 32:64] = 2.0 ** 7                          # an exact power of two
    c[3, 64:96] = np.ldexp(1.0, 200)                # beyond the largest scale: X clamps to 127
    v, codes, scale = codecs.mxfp4_quantize(c)
    assert codes.dtype == np.uint8 and scale.shape == (n, D // 32)
    for i in range(n):
        for b in range(D // 32):
            blk = c[i, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            X = -127 if amax == 0 else min(max(_scale_exp_brute(amax) - 2, -127), 127)
            assert scale[i, b] == X + 127, (i, b)
            want = _nearest_e2m1_brute(blk / 2.0 ** X) * 2.0 ** X
            assert np.array_equal(v[i, 32 * b:32 * b + 32], want), (i, b)
            if amax > 0 and X < 127:
                # the largest magnitude maps into [4, 8) before rounding: element 4 or 6
                assert np.abs(want).max() / 2.0 ** X in (4.0, 6.0)
    assert np.array_equal(codecs.mxfp4_dequantize(codes, scale), v)
    assert np.all(scale[0] == 0) and np.all(v[0] == 0)
    assert scale[2, 1] == 7 - 2 + 127 and np.all(v[2, 32:64] == 2.0 ** 7)
    assert scale[3, 2] == 254 and np.all(v[3, 64:96] == 6.0 * 2.0 ** 127)
