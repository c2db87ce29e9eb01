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
