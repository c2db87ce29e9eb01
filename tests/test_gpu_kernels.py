"""GPU parity of each HIP call against the oracle on the same seeded inputs.

Sizes span several tiles/blocks and ragged tails; rows cover the edge cases of
the visibility rule (no visible entry, one entry, short windows at t < W)."""
import math

import numpy as np
import pytest
import torch

from oracle import codecs, method
from tests.compare import assert_close, assert_scores_close, bf16_code_flips, e4m3_flips, mxfp4_flips, topk_parity
from tests.gpu_util import DEV, dev, dev_codes, dev_i32, host, rng_store

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("sequence_compressed_kv_amd")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.load()


# ---------------------------------------------------------------- compression
COMPRESS_CASES = [
    # m, o, D, in, out, scaled, B, N
    (4, 4, 64, "f32", "f32", False, 1, 4096),
    (4, 4, 32, "f32", "f32", False, 1, 4096),
    (128, 0, 128, "bf16", "bf16", False, 2, 8192),
    (4, 4, 512, "bf16", "bf16", False, 1, 2048),
    (4, 4, 512, "bf16", "e4m3", True, 1, 2048),
    (4, 4, 128, "bf16", "e4m3", False, 2, 1024),
    (128, 0, 512, "bf16", "e4m3", True, 1, 16384),
    (4, 4, 8, "bf16", "bf16", False, 3, 203),
    (2, 6, 16, "f32", "bf16", False, 2, 101),
]
# key-tile output (the indexer stream): in, out, D, B, N
TILED_CASES = [("bf16", "bf16", 128, 2, 4096), ("bf16", "e4m3", 128, 1, 1024), ("f32", "f32", 32, 1, 4096),
               ("bf16", "bf16", 64, 1, 520)]


@pytest.mark.parametrize("m,o,D,ins,outs,scaled,B,N", COMPRESS_CASES)
def test_compress_parity(m, o, D, ins, outs, scaled, B, N):
    print(f"compress m={m} o={o} D={D} {ins}->{outs} scaled={scaled} B={B} N={N}", flush=True)
    rng = np.random.default_rng(100 + D + m)
    v = rng_store(rng, (B, N, D), ins)
    g = rng_store(rng, (B, N, D), ins, 2.0)
    bpos = rng.normal(0, 0.5, (m + o, D)).astype(np.float32)
    E = N // m
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}[outs]
    out = torch.zeros(B, E, D, device=DEV, dtype=odt if outs != "e4m3" else torch.uint8)
    if outs == "e4m3":
        out = out.view(torch.float8_e4m3fn)
    osc = torch.zeros(B, E, device=DEV, dtype=torch.float32) if scaled else None
    pool = sk.Pool(dev(v, ins), dev(g, ins), dev(bpos), out, osc)
    if m == 128:
        sk.hca_compress(pool, m=m, o=o)
    else:
        sk.csa_compress(pool, m=m, o=o)
    torch.cuda.synchronize()
    for b in range(B):
        c = method.compress(v[b], g[b], bpos, m, o)
        # same softmax weights on |v|: the scale of the fp32 rounding error of each pooled sum
        mag = method.compress(np.abs(v[b]), g[b], bpos, m, o)
        if outs == "f32":
            assert_close(host(out[b]), c, rtol=1e-5, what="f32 entries")
        elif outs == "bf16":
            st = method.store_entries(c, "bf16")
            n_bad, n_unexplained = bf16_code_flips(host(out[b]), c, st["values"], magnitude=mag)
            assert n_unexplained == 0, f"{n_unexplained} of {n_bad} bf16 codes differ"
        else:
            st = method.store_entries(c, "e4m3") if scaled else method.store_keys(c, "e4m3")
            gc = host(out[b])
            if scaled:
                gs = osc[b].cpu().numpy().astype(np.float64)
                np.testing.assert_allclose(gs, st["scale"], rtol=2e-6)
                y, ymag = c / st["scale"][:, None], mag / st["scale"][:, None]
            else:
                y, ymag = c, mag
            n_bad, n_unexplained = e4m3_flips(gc, st["codes"], y, ymag)
            assert n_unexplained == 0, f"{n_unexplained} of {n_bad} e4m3 codes differ"


@pytest.mark.parametrize("ins,outs,D,B,N", TILED_CASES)
def test_compress_key_tiles(ins, outs, D, B, N):
    """The indexer stream written in the tiled key layout holds the same values as the rows layout."""
    print(f"compress key tiles {ins}->{outs} D={D} B={B} N={N}", flush=True)
    rng = np.random.default_rng(7 + D)
    v, g = rng_store(rng, (B, N, D), ins), rng_store(rng, (B, N, D), ins, 2.0)
    bpos = rng.normal(0, 0.5, (8, D)).astype(np.float32)
    E = N // 4
    Ec = (E + 31) // 32 * 32
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}[outs]
    rows = torch.zeros(B, Ec, D, device=DEV, dtype=tdt)
    tiles = torch.zeros(B, Ec // 32, D // 8, 32, 8, device=DEV, dtype=tdt)
    if outs == "e4m3":
        rows, tiles = rows.view(torch.float8_e4m3fn), tiles.view(torch.float8_e4m3fn)
    vd, gd, bd = dev(v, ins), dev(g, ins), dev(bpos)
    sk.csa_compress(sk.Pool(vd, gd, bd, rows), sk.Pool(vd, gd, bd, tiles, layout=sk.LAYOUT_KEY_TILES), m=4, o=4)
    torch.cuda.synchronize()
    back = sk.from_key_tiles(tiles)
    if outs == "e4m3":
        assert torch.equal(back.view(torch.uint8), rows.view(torch.uint8))
    else:
        assert torch.equal(back, rows)
    # and the rows themselves follow the oracle
    for b in range(B):
        c = method.compress(v[b], g[b], bpos, 4, 4)
        mag = method.compress(np.abs(v[b]), g[b], bpos, 4, 4)
        got = host(rows[b])[:E]
        if outs == "f32":
            assert_close(got, c, rtol=1e-5, what="f32 keys")
        elif outs == "bf16":
            assert bf16_code_flips(got, c, method.store_keys(c, "bf16")["values"], magnitude=mag)[1] == 0
        else:
            st = method.store_keys(c, "e4m3")
            assert e4m3_flips(got, st["codes"], c, mag)[1] == 0


@pytest.mark.parametrize("ins,D,B,N", [("bf16", 128, 2, 4096), ("f32", 64, 1, 1030), ("bf16", 32, 1, 600),
                                       ("bf16", 256, 1, 700), ("f32", 512, 1, 520)])
def test_compress_mxfp4_keys(ins, D, B, N):
    """FP4 indexer keys: the GPU's MXFP4 blocks against the oracle's, block scales and
    e2m1 codes, with flips only where the fp32 pooling error can cross a rounding
    boundary or a power of two."""
    print(f"compress mxfp4 keys {ins} D={D} B={B} N={N}", flush=True)
    rng = np.random.default_rng(17 + D + N)
    v, g = rng_store(rng, (B, N, D), ins), rng_store(rng, (B, N, D), ins, 2.0)
    v[:, :8] = 0.0                                   # zero tokens: the first entry's blocks are all zero
    bpos = rng.normal(0, 0.5, (8, D)).astype(np.float32)
    E = N // 4
    keys = sk.Mxfp4Keys.empty(B, (E + 31) // 32 * 32, D, DEV)
    keys.tiles.fill_(0x5A)
    vd, gd, bd = dev(v, ins), dev(g, ins), dev(bpos)
    sk.csa_compress(sk.Pool(vd, gd, bd, keys, layout=sk.LAYOUT_KEY_TILES), m=4, o=4)
    torch.cuda.synchronize()
    codes, scale = (t.cpu().numpy() for t in sk.mxfp4_unpack(keys))
    for b in range(B):
        c = method.compress(v[b], g[b], bpos, 4, 4)
        mag = method.compress(np.abs(v[b]), g[b], bpos, 4, 4)
        n_diff, n_un = mxfp4_flips(codes[b, :E], scale[b, :E], c, mag)
        assert n_un == 0, f"seq {b}: {n_un} of {n_diff} MXFP4 scales/codes unexplained"
        assert n_diff <= 1e-3 * E * D, f"seq {b}: {n_diff} flips"
        st = method.store_keys(c, "mxfp4")
        assert np.all(scale[b, 0] == 0) and np.all(st["scale"][0] == 0)          # the all-zero entry


APPEND_CASES = [
    # m, o, D, in, out, scaled, key tiles, B, N, ring slots P
    (4, 4, 64, "bf16", "bf16", False, False, 3, 600, 8),
    (4, 4, 128, "bf16", "bf16", False, True, 2, 520, 8),          # indexer keys, tiled
    (4, 4, 128, "bf16", "e4m3", False, True, 2, 300, 8),          # unscaled e4m3 keys, tiled
    (4, 4, 512, "bf16", "e4m3", True, False, 2, 300, 128),        # latent: the window ring as value ring
    (128, 0, 64, "f32", "f32", False, False, 2, 700, 128),
    (128, 0, 512, "bf16", "e4m3", True, False, 1, 520, 128),
    (2, 6, 16, "f32", "bf16", False, False, 2, 101, 9),
]


@pytest.mark.parametrize("m,o,D,ins,outs,scaled,tiled,B,N,P", APPEND_CASES)
def test_append_token_by_token(m, o, D, ins, outs, scaled, tiled, B, N, P):
    """Decode appends, one token per call, with the sequences at different
    positions: the entries equal the bulk compressor's bit for bit (and follow the
    oracle in code space), and the rings hold each sequence's last P tokens."""
    print(f"append m={m} o={o} D={D} {ins}->{outs} scaled={scaled} tiled={tiled} B={B} N={N} P={P}", flush=True)
    rng = np.random.default_rng(300 + D + m + N)
    v = rng_store(rng, (B, N, D), ins)
    g = rng_store(rng, (B, N, D), ins, 2.0)
    bpos = rng.normal(0, 0.5, (m + o, D)).astype(np.float32)
    E = N // m
    E_cap = (E + 31) // 32 * 32 if tiled else E
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}[outs]

    def cache():
        t = (torch.zeros(B, E_cap // 32, D // 8, 32, 8, device=DEV, dtype=tdt) if tiled
             else torch.zeros(B, E_cap, D, device=DEV, dtype=tdt))
        return t.view(torch.float8_e4m3fn) if outs == "e4m3" else t

    out_a, out_b = cache(), cache()
    sc_a = torch.zeros(B, E_cap, device=DEV) if scaled else None
    sc_b = torch.zeros(B, E_cap, device=DEV) if scaled else None
    layout = sk.LAYOUT_KEY_TILES if tiled else sk.LAYOUT_ROWS
    vd, gd, bd = dev(v, ins), dev(g, ins), dev(bpos)
    rv = torch.zeros(B, P, D, device=DEV, dtype=vd.dtype)
    rg = torch.zeros(B, P, D, device=DEV, dtype=vd.dtype)
    off = [3 * b for b in range(B)]                          # sequence b starts 3b calls late
    ar = torch.arange(B, device=DEV)
    for c in range(N + max(off)):
        p_host = [c - off[b] if 0 <= c - off[b] < N else -1 for b in range(B)]
        pos = dev_i32(p_host)
        pc = pos.clamp(min=0).long()
        a = sk.Append(pos, vd[ar, pc].contiguous(), gd[ar, pc].contiguous(), rv, rg, bd, out_a, sc_a, layout)
        if m == 128:
            sk.hca_append(a, m=m, o=o)
        else:
            sk.csa_append(a, m=m, o=o)
    bulk = sk.Pool(vd, gd, bd, out_b, sc_b, layout)
    if m == 128:
        sk.hca_compress(bulk, m=m, o=o)
    else:
        sk.csa_compress(bulk, m=m, o=o)
    torch.cuda.synchronize()
    raw = (lambda t: t.view(torch.uint8)) if outs == "e4m3" else (lambda t: t)
    assert torch.equal(raw(out_a), raw(out_b)), "appended entries differ from the bulk compressor's"
    if scaled:
        assert torch.equal(sc_a, sc_b)
    for b in range(B):                                       # the rings: the last P tokens, slot = position mod P
        last = np.arange(N - P, N)
        np.testing.assert_array_equal(host(rv[b])[last % P], v[b][last])
        np.testing.assert_array_equal(host(rg[b])[last % P], g[b][last])
    # the oracle, in code space, for sequence 0
    c = method.compress(v[0], g[0], bpos, m, o)
    mag = method.compress(np.abs(v[0]), g[0], bpos, m, o)
    got = host(sk.from_key_tiles(out_a) if tiled else out_a)[0][:E]
    if outs == "f32":
        assert_close(got, c, rtol=1e-5, what="f32 entries")
    elif outs == "bf16":
        st = method.store_keys(c, "bf16") if tiled else method.store_entries(c, "bf16")
        assert bf16_code_flips(got, c, st["values"], magnitude=mag)[1] == 0
    else:
        st = method.store_entries(c, "e4m3") if scaled else method.store_keys(c, "e4m3")
        if scaled:
            gs = sc_a[0].cpu().numpy().astype(np.float64)[:E]
            np.testing.assert_allclose(gs, st["scale"], rtol=2e-6)
            y, ymag = c / st["scale"][:, None], mag / st["scale"][:, None]
        else:
            y, ymag = c, mag
        assert e4m3_flips(got, st["codes"], y, ymag)[1] == 0


def test_append_mxfp4_keys_match_bulk():
    """MXFP4 indexer keys appended token by token equal the bulk compressor's tiles
    byte for byte (entries whose window is complete)."""
    B, N, D, P = 2, 300, 128, 8
    print(f"append mxfp4 B={B} N={N} D={D}", flush=True)
    rng = np.random.default_rng(41)
    v, g = rng_store(rng, (B, N, D), "bf16"), rng_store(rng, (B, N, D), "bf16", 2.0)
    bpos = rng.normal(0, 0.5, (8, D)).astype(np.float32)
    E = N // 4
    E_cap = (E + 31) // 32 * 32
    vd, gd, bd = dev(v, "bf16"), dev(g, "bf16"), dev(bpos)
    ka, kb = sk.Mxfp4Keys.empty(B, E_cap, D, DEV), sk.Mxfp4Keys.empty(B, E_cap, D, DEV)
    ka.tiles.zero_()
    kb.tiles.zero_()
    rv = torch.zeros(B, P, D, device=DEV, dtype=vd.dtype)
    rg = torch.zeros(B, P, D, device=DEV, dtype=vd.dtype)
    ar = torch.arange(B, device=DEV)
    for t in range(N):
        pos = dev_i32([t] * B)
        sk.csa_append(sk.Append(pos, vd[ar, t].contiguous(), gd[ar, t].contiguous(), rv, rg, bd, ka,
                                layout=sk.LAYOUT_KEY_TILES), m=4, o=4)
    sk.csa_compress(sk.Pool(vd, gd, bd, kb, layout=sk.LAYOUT_KEY_TILES), m=4, o=4)
    torch.cuda.synchronize()
    assert torch.equal(ka.tiles, kb.tiles)


@pytest.mark.parametrize("kv_out,scaled", [("bf16", False), ("e4m3", True)])
def test_csa_append_two_streams(kv_out, scaled):
    """csa_append with the latent and the indexer stream (one launch when their
    dtypes agree, two otherwise) equals csa_compress of both streams bit for bit."""
    print(f"csa append, two streams: kv -> {kv_out} scaled={scaled}", flush=True)
    rng = np.random.default_rng(41)
    B, N, D, DI, P = 2, 264, 512, 128, 128
    v, g = rng_store(rng, (B, N, D), "bf16"), rng_store(rng, (B, N, D), "bf16", 2.0)
    vI, gI = rng_store(rng, (B, N, DI), "bf16"), rng_store(rng, (B, N, DI), "bf16", 2.0)
    bp, bpI = rng.normal(0, 0.5, (8, D)).astype(np.float32), rng.normal(0, 0.5, (8, DI)).astype(np.float32)
    E = N // 4
    Ec = (E + 31) // 32 * 32
    kdt = torch.bfloat16 if kv_out == "bf16" else torch.uint8

    def caches():
        ent = torch.zeros(B, E, D, device=DEV, dtype=kdt)
        ent = ent.view(torch.float8_e4m3fn) if kv_out == "e4m3" else ent
        scale = torch.zeros(B, E, device=DEV) if scaled else None
        return ent, scale, sk.key_tiles_empty(B, Ec, DI, torch.bfloat16, DEV).zero_()

    (ea, sa, ka), (eb, sb, kb) = caches(), caches()
    vd, gd, vId, gId, bd, bId = dev(v, "bf16"), dev(g, "bf16"), dev(vI, "bf16"), dev(gI, "bf16"), dev(bp), dev(bpI)
    rv, rg = (torch.zeros(B, P, D, device=DEV, dtype=torch.bfloat16) for _ in range(2))
    rvI, rgI = (torch.zeros(B, 8, DI, device=DEV, dtype=torch.bfloat16) for _ in range(2))
    for t in range(N):
        pos = dev_i32([t] * B)
        sk.csa_append(sk.Append(pos, vd[:, t].contiguous(), gd[:, t].contiguous(), rv, rg, bd, ea, sa),
                      sk.Append(pos, vId[:, t].contiguous(), gId[:, t].contiguous(), rvI, rgI, bId, ka,
                                layout=sk.LAYOUT_KEY_TILES), m=4, o=4)
    sk.csa_compress(sk.Pool(vd, gd, bd, eb, sb), sk.Pool(vId, gId, bId, kb, layout=sk.LAYOUT_KEY_TILES), m=4, o=4)
    torch.cuda.synchronize()
    raw = (lambda x: x.view(torch.uint8)) if kv_out == "e4m3" else (lambda x: x)
    assert torch.equal(raw(ea), raw(eb))
    assert torch.equal(ka, kb)
    if scaled:
        assert torch.equal(sa, sb)


# input, latent output ("e4m3s": scaled e4m3), key output, latent dim, key dim, keys tiled, tokens,
# first entry, entries (None: the rest), a latent channel with a wide bias spread
PAIR_CASES = [
    ("bf16", "bf16", "bf16", 512, 128, True, 40000, 0, None, False),      # the 128K layer's types, J > 1
    ("bf16", "bf16", "bf16", 512, 128, True, 20000, 1001, 3000, True),    # an entry range, online-path channel
    ("bf16", "e4m3s", "e4m3", 512, 128, True, 30000, 0, None, False),     # the 1M layer's types
    ("bf16", "e4m3s", "e4m3s", 512, 128, False, 9000, 7, 2000, False),
    ("bf16", "bf16", "mxfp4", 512, 128, True, 12000, 0, None, True),      # MXFP4 indexer keys
    ("bf16", "e4m3s", "mxfp4", 256, 64, True, 8000, 33, 1500, False),
    ("f32", "f32", "f32", 256, 64, False, 6000, 0, None, False),          # no pair instance: two launches
]


def _pool_out(B, E, D, kind, tiled):
    """(cache, scale or None, raw-bytes view) for one stream's output kind."""
    if kind == "mxfp4":
        keys = sk.Mxfp4Keys.empty(B, (E + 31) // 32 * 32, D, DEV)
        keys.tiles.zero_()
        return keys, None, lambda: keys.tiles
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "e4m3": torch.uint8, "e4m3s": torch.uint8}[kind]
    if tiled:
        t = sk.key_tiles_empty(B, (E + 31) // 32 * 32, D, dt, DEV).zero_()
    else:
        t = torch.zeros(B, E, D, device=DEV, dtype=dt)
    out = t.view(torch.float8_e4m3fn) if kind.startswith("e4m3") else t
    sc = torch.zeros(B, E, device=DEV) if kind == "e4m3s" else None
    return out, sc, lambda: t


@pytest.mark.parametrize("ins,out0,out1,D,DI,tiled,N,e_begin,e_count,spread", PAIR_CASES)
def test_csa_compress_pair_equals_single_streams(ins, out0, out1, D, DI, tiled, N, e_begin, e_count, spread):
    """csa_compress with both streams runs them in one grid where a pair instance
    exists for their types; its entries equal those of two single-stream calls
    bit for bit (so the single stream's parity with the oracle carries over)."""
    print(f"compress pair {ins} -> {out0} + {out1} D={D} DI={DI} N={N} range={e_begin}+{e_count} "
          f"spread={spread}", flush=True)
    rng = np.random.default_rng(N + D + e_begin)
    B, m, o = 2, 4, 4
    v, g = rng_store(rng, (B, N, D), ins), rng_store(rng, (B, N, D), ins, 2.0)
    vI, gI = rng_store(rng, (B, N, DI), ins), rng_store(rng, (B, N, DI), ins, 2.0)
    bp, bpI = rng.normal(0, 0.5, (8, D)).astype(np.float32), rng.normal(0, 0.5, (8, DI)).astype(np.float32)
    if spread:
        bp[0, 5], bp[7, 5] = 35.0, -35.0                            # this channel takes the online path
    E = N // m
    n = E - e_begin if e_count is None else e_count
    vd, gd, vId, gId, bd, bId = dev(v, ins), dev(g, ins), dev(vI, ins), dev(gI, ins), dev(bp), dev(bpI)
    lay = sk.LAYOUT_KEY_TILES if tiled or out1 == "mxfp4" else sk.LAYOUT_ROWS
    (ea, sa, ra), (ka, saI, rka) = _pool_out(B, E, D, out0, False), _pool_out(B, E, DI, out1, tiled)
    (eb, sb, rb), (kb, sbI, rkb) = _pool_out(B, E, D, out0, False), _pool_out(B, E, DI, out1, tiled)
    args = dict(m=m, o=o, e_begin=e_begin, e_count=n)
    sk.csa_compress(sk.Pool(vd, gd, bd, ea, sa), sk.Pool(vId, gId, bId, ka, saI, layout=lay), **args)
    sk.csa_compress(sk.Pool(vd, gd, bd, eb, sb), **args)
    sk.csa_compress(sk.Pool(vId, gId, bId, kb, sbI, layout=lay), **args)
    torch.cuda.synchronize()
    assert torch.equal(ra(), rb()), "latent entries of the paired launch differ"
    assert torch.equal(rka(), rkb()), "indexer keys of the paired launch differ"
    for x, y in ((sa, sb), (saI, sbI)):
        if x is not None:
            assert torch.equal(x, y)
    assert ra()[:, e_begin:e_begin + n].float().abs().sum() > 0        # the range was written


@pytest.mark.parametrize("D,outs,scaled", [(64, "bf16", False), (512, "e4m3", True)])
def test_overlap_windows_with_wide_bias_spread(D, outs, scaled):
    """4:1 overlapping windows whose position biases spread by more than 60 in some
    channels (those entries take the online softmax): bulk and token-by-token
    appends store the same bits, and both follow the oracle in code space."""
    print(f"wide bias spread D={D} {outs} scaled={scaled}", flush=True)
    rng = np.random.default_rng(41 + D)
    B, N, P, m, o = 2, 160, 8, 4, 4
    v = rng_store(rng, (B, N, D), "bf16")
    g = rng_store(rng, (B, N, D), "bf16", 2.0)
    bpos = rng.normal(0, 0.5, (m + o, D)).astype(np.float32)
    bpos[0, 3], bpos[7, 3] = 33.0, -33.0                       # channel 3: spread 66
    if D > 64:
        bpos[2, D - 5], bpos[5, D - 5] = -40.0, 25.0           # a channel in the last lane group
    E = N // m
    tdt = torch.uint8 if outs == "e4m3" else torch.bfloat16
    mk = (lambda: torch.zeros(B, E, D, device=DEV, dtype=tdt).view(torch.float8_e4m3fn)) if outs == "e4m3" else \
        (lambda: torch.zeros(B, E, D, device=DEV, dtype=tdt))
    out_a, out_b = mk(), mk()
    sc_a = torch.zeros(B, E, device=DEV) if scaled else None
    sc_b = torch.zeros(B, E, device=DEV) if scaled else None
    vd, gd, bd = dev(v, "bf16"), dev(g, "bf16"), dev(bpos)
    rv = torch.zeros(B, P, D, device=DEV, dtype=vd.dtype)
    rg = torch.zeros(B, P, D, device=DEV, dtype=vd.dtype)
    ar = torch.arange(B, device=DEV)
    for c in range(N):
        pos = dev_i32([c] * B)
        a = sk.Append(pos, vd[ar, pos.long()].contiguous(), gd[ar, pos.long()].contiguous(), rv, rg, bd, out_a, sc_a)
        sk.csa_append(a, m=m, o=o)
    sk.csa_compress(sk.Pool(vd, gd, bd, out_b, sc_b), m=m, o=o)
    torch.cuda.synchronize()
    raw = (lambda t: t.view(torch.uint8)) if outs == "e4m3" else (lambda t: t)
    assert torch.equal(raw(out_a), raw(out_b)), "appended entries differ from the bulk compressor's"
    if scaled:
        assert torch.equal(sc_a, sc_b)
    for b in range(B):
        c = method.compress(v[b], g[b], bpos, m, o)
        mag = method.compress(np.abs(v[b]), g[b], bpos, m, o)
        got = host(out_b[b])
        if outs == "bf16":
            st = method.store_entries(c, "bf16")
            assert bf16_code_flips(got, c, st["values"], magnitude=mag)[1] == 0
        else:
            st = method.store_entries(c, "e4m3")
            np.testing.assert_allclose(sc_b[b].cpu().numpy().astype(np.float64), st["scale"], rtol=2e-6)
            assert e4m3_flips(got, st["codes"], c / st["scale"][:, None], mag / st["scale"][:, None])[1] == 0


@pytest.mark.parametrize("D,outs,e_begin,e_count", [(512, "bf16", 777, 9000), (128, "e4m3", 4099, 33000)])
def test_overlap_range_equals_whole_sequence(D, outs, e_begin, e_count):
    """A range of entries starting mid-sequence, long enough that every block of the
    4:1 compressor pools a run of several steps (the first-half sums handed from
    slot to slot and across steps): the entries equal those of one call over the
    whole sequence bit for bit, the entries outside the range stay untouched, and
    sampled entries follow the oracle in code space."""
    print(f"overlap range D={D} {outs} e_begin={e_begin} e_count={e_count}", flush=True)
    rng = np.random.default_rng(9 + D)
    E = e_begin + e_count + 300
    N = 4 * E
    v = rng_store(rng, (1, N, D), "bf16")
    g = rng_store(rng, (1, N, D), "bf16", 2.0)
    bpos = rng.normal(0, 0.5, (8, D)).astype(np.float32)
    vd, gd, bd = dev(v, "bf16"), dev(g, "bf16"), dev(bpos)
    if outs == "e4m3":
        whole = torch.zeros(1, E, D, device=DEV, dtype=torch.uint8).view(torch.float8_e4m3fn)
        part = torch.full((1, E, D), 0x5A, device=DEV, dtype=torch.uint8).view(torch.float8_e4m3fn)
    else:
        whole = torch.zeros(1, E, D, device=DEV, dtype=torch.bfloat16)
        part = torch.full((1, E, D), 7.0, device=DEV, dtype=torch.bfloat16)
    sk.csa_compress(sk.Pool(vd, gd, bd, whole), m=4, o=4)
    sk.csa_compress(sk.Pool(vd, gd, bd, part), m=4, o=4, e_begin=e_begin, e_count=e_count)
    torch.cuda.synchronize()
    raw = (lambda t: t.view(torch.uint8)) if outs == "e4m3" else (lambda t: t)
    lo, hi = e_begin, e_begin + e_count
    assert torch.equal(raw(part)[:, lo:hi], raw(whole)[:, lo:hi]), "a range differs from the whole-sequence call"
    untouched = 0x5A if outs == "e4m3" else 7.0
    assert bool((raw(part)[:, :lo] == untouched).all()) and bool((raw(part)[:, hi:] == untouched).all())
    sample = np.unique(np.concatenate([np.arange(lo, lo + 70), rng.integers(lo, hi, 200), np.arange(hi - 70, hi)]))
    t0, t1 = 4 * (int(sample.min()) - 1), 4 * int(sample.max()) + 4
    c_all = method.compress(v[0, t0:t1], g[0, t0:t1], bpos, 4, 4)
    m_all = method.compress(np.abs(v[0, t0:t1]), g[0, t0:t1], bpos, 4, 4)
    off = t0 // 4
    c, mag = c_all[sample - off], m_all[sample - off]
    got = host(whole[0])[sample]
    if outs == "bf16":
        assert bf16_code_flips(got, c, method.store_entries(c, "bf16")["values"], magnitude=mag)[1] == 0
    else:
        st = method.store_keys(c, "e4m3")
        assert e4m3_flips(got, st["codes"], c, mag)[1] == 0


def test_compress_appends_only_requested_entries():
    rng = np.random.default_rng(5)
    B, N, D = 2, 256, 64
    v, g = rng_store(rng, (B, N, D), "bf16"), rng_store(rng, (B, N, D), "bf16")
    bpos = rng.normal(0, 0.5, (8, D)).astype(np.float32)
    out = torch.full((B, 64, D), 7.0, device=DEV, dtype=torch.bfloat16)
    sk.csa_compress(sk.Pool(dev(v, "bf16"), dev(g, "bf16"), dev(bpos), out), m=4, o=4, e_begin=5, e_count=9)
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(o[:, :5] == 7.0) and np.all(o[:, 14:] == 7.0)
    for b in range(B):
        c = method.compress(v[b], g[b], bpos, 4, 4)[5:14]
        mag = method.compress(np.abs(v[b]), g[b], bpos, 4, 4)[5:14]
        n_bad, n_un = bf16_code_flips(o[b, 5:14], c, method.store_entries(c, "bf16")["values"], magnitude=mag)
        assert n_un == 0


# ---------------------------------------------------------------- indexer + top-k (decode rows)
INDEX_CASES = [
    # keys, H_I, D_I, E_cap, positions, k
    ("f32", 4, 32, 1024, [4095], 64),
    ("bf16", 64, 128, 4096, [16511, 5000, 131, 127, 132, 600], 256),
    ("e4m3", 64, 128, 4096, [16511, 9000], 1024),
    ("bf16", 32, 64, 2000, [8127, 4000], 100),
    ("bf16", 64, 128, 40000, [160127], 1024),
    ("bf16", 64, 128, 70000, [279999, 200000], 2048),
    ("e4m3", 64, 128, 70000, [279999], 100),
    ("mxfp4", 64, 128, 4096, [16511, 9000, 131, 600], 1024),
    ("mxfp4", 32, 64, 2000, [8127, 4000], 100),
    ("mxfp4", 64, 128, 70000, [279999], 2048),
    # 40 rows over a 32K-entry cache: rows cut into 8192-entry slices, ragged row lengths
    ("bf16", 32, 64, 32768, [131071 - 997 * i for i in range(40)], 512),
]


def _index_inputs(rng, keys_s, HI, DI, B, E_cap):
    qs = "f32" if keys_s == "f32" else "bf16"
    q = rng_store(rng, (B, HI, DI), qs)
    w = rng.normal(0, 1, (B, HI)).astype(np.float32)
    if keys_s == "mxfp4":
        # per-key magnitudes spread over a few binades, so blocks take different scales
        raw = rng.normal(0, 1, (B * E_cap, DI)) * np.ldexp(1.0, rng.integers(-3, 4, size=(B * E_cap, 1)))
        vals, codes, scale = codecs.mxfp4_quantize(raw)
        kv = vals.reshape(B, E_cap, DI)
        keys = sk.mxfp4_pack(torch.from_numpy(codes.reshape(B, E_cap, DI)),
                             torch.from_numpy(scale.reshape(B, E_cap, DI // 32)))
        return q, w, kv, dev(q, qs), dev(w), sk.Mxfp4Keys(keys.tiles.to(DEV), DI)
    if keys_s == "e4m3":
        kv = codecs.round_e4m3(rng.normal(0, 1, (B, E_cap, DI)))
        keys_dev = dev_codes(codecs.e4m3_encode(kv))
    else:
        kv = rng_store(rng, (B, E_cap, DI), keys_s)
        keys_dev = dev(kv, keys_s)
    # the indexer reads keys in the tiled layout
    return q, w, kv.astype(np.float64), dev(q, qs), dev(w), sk.to_key_tiles(keys_dev)


@pytest.mark.parametrize("keys_s,HI,DI,E_cap,positions,k", INDEX_CASES)
def test_index_topk_decode(keys_s, HI, DI, E_cap, positions, k):
    print(f"index decode {keys_s} H_I={HI} D_I={DI} E_cap={E_cap} pos={positions} k={k}", flush=True)
    rng = np.random.default_rng(E_cap + k)
    B = len(positions)
    q, w, kv, qd, wd, keysd = _index_inputs(rng, keys_s, HI, DI, B, E_cap)
    pos = dev_i32(positions)
    rows = sk.RowSpec.decode(pos, max(positions))
    out_idx = torch.full((B, k), -7, device=DEV, dtype=torch.int32)
    out_score = torch.zeros(B, k, device=DEV, dtype=torch.float32)
    cover = min(method.entries_visible(max(positions), 4, 128), E_cap)
    scores = torch.full((B, max(cover, 1)), float("nan"), device=DEV, dtype=torch.float32)
    sk.csa_index_score(rows, qd, wd, keysd, scores, m=4, W=128, k=k)
    sk.csa_index_topk(rows, qd, wd, keysd, out_idx, m=4, W=128, k=k, out_score=out_score)
    torch.cuda.synchronize()
    gi, gsc, gs = host(out_idx), host(out_score), host(scores)
    for r, t in enumerate(positions):
        ev = min(method.entries_visible(t, 4, 128), E_cap)
        s = method.index_scores(q[r], w[r], kv[r, :ev])
        if ev:
            assert_scores_close(gs[r, :ev], s, q[r], w[r], kv[r, :ev], rtol=2e-6, what=f"scores row {r}")
        ok, msg = topk_parity(gi[r], method.topk(s, k), s)
        assert ok, f"row {r} (t={t}, E_vis={ev}): {msg}"
        sel = gi[r][gi[r] >= 0]
        np.testing.assert_array_equal(gsc[r, :len(sel)], gs[r, sel])
        assert np.all(np.isneginf(gsc[r, len(sel):]))


@pytest.mark.parametrize("case", ["all_tied", "zeros", "hot_region", "band_tied", "mixed_rows"])
def test_index_topk_decode_hint_edges(case):
    """Decode rows long enough for the selection to filter by the scoring kernel's
    per-wave hint, with scores set exactly: a unit query on key dimension 0 and
    one head weight make s_j = ReLU(k_j[0]).  Every score tied (the survivors
    overflow the final block, which streams the row), mostly zeros (ties at 0), a
    region of high scores (many survivors from one part of the row), a band tied
    near the threshold, and rows whose waves hold too few keys for the bound (a
    short row, an empty row, a row with k above its visible count)."""
    print(f"index decode hint edge case {case}", flush=True)
    rng = np.random.default_rng(abs(hash(case)) % 2**32)
    E_cap, HI, DI, k = 70016, 64, 128, 2048
    pos = [4 * 70000 + 131] * 3
    if case == "mixed_rows":
        pos = [4 * 70000 + 131, 4 * 1500 + 131, 100, 4 * 1800 + 131]
    B = len(pos)
    x0 = rng.normal(0, 1, (B, E_cap))
    if case == "all_tied":
        x0[:] = 1.5
    elif case == "zeros":
        x0[:] = -1.0
        x0[:, rng.choice(E_cap, size=500, replace=False)] = rng.uniform(0.5, 2.0, (B, 500))
    elif case == "hot_region":
        x0[:, 30000:38192] += 5.0
    elif case == "band_tied":
        x0[:, rng.choice(E_cap, size=E_cap // 3, replace=False)] = 1.875
    kv = rng_store(rng, (B, E_cap, DI), "bf16")
    kv[:, :, 0] = torch.from_numpy(x0.astype(np.float32)).to(torch.bfloat16).float().numpy()
    q = np.zeros((B, HI, DI), np.float32)
    q[:, 0, 0] = 1.0
    w = np.zeros((B, HI), np.float32)
    w[:, 0] = 1.0
    rows = sk.RowSpec.decode(dev_i32(pos), max(pos))
    out_idx = torch.full((B, k), -7, device=DEV, dtype=torch.int32)
    out_score = torch.zeros(B, k, device=DEV, dtype=torch.float32)
    keys = sk.to_key_tiles(dev(kv, "bf16"))
    sk.csa_index_topk(rows, dev(q, "bf16"), dev(w), keys, out_idx, m=4, W=128, k=k, out_score=out_score)
    torch.cuda.synchronize()
    gi, gsc = host(out_idx), host(out_score)
    for r, t in enumerate(pos):
        ev = min(method.entries_visible(t, 4, 128), E_cap)
        s = method.index_scores(q[r], w[r], kv[r, :ev].astype(np.float64))
        np.testing.assert_array_equal(s, np.maximum(kv[r, :ev, 0].astype(np.float64), 0.0))
        ora = method.topk(s, k)
        np.testing.assert_array_equal(gi[r], ora, err_msg=f"{case} row {r} (t={t}, E_vis={ev})")
        sel = gi[r][gi[r] >= 0]
        np.testing.assert_array_equal(gsc[r, :len(sel)], s[sel].astype(np.float32))


CAUSAL_CASES = [
    ("bf16", 64, 128, 800, 3300, 64),
    ("f32", 4, 32, 300, 1300, 16),
    ("e4m3", 64, 128, 600, 2500, 128),
    ("bf16", 32, 64, 700, 2900, 32),
    ("e4m3", 64, 64, 500, 2123, 64),
    ("mxfp4", 64, 128, 800, 3300, 64),
    ("mxfp4", 32, 64, 700, 2900, 32),
]


@pytest.mark.parametrize("keys_s,HI,DI,E_cap,T,k", CAUSAL_CASES)
def test_index_topk_causal(keys_s, HI, DI, E_cap, T, k):
    print(f"index causal {keys_s} H_I={HI} D_I={DI} E_cap={E_cap} T={T} k={k}", flush=True)
    rng = np.random.default_rng(T + k)
    qs = "f32" if keys_s == "f32" else "bf16"
    q = rng_store(rng, (T, HI, DI), qs)
    w = rng.normal(0, 1, (T, HI)).astype(np.float32)
    _, _, kv, _, _, keysd = _index_inputs(rng, keys_s, HI, DI, 1, E_cap)
    rows = sk.RowSpec.causal(T)
    out_idx = torch.full((T, k), -7, device=DEV, dtype=torch.int32)
    cover = min(method.entries_visible(T - 1, 4, 128), E_cap)
    scores = torch.full((T, cover + 5), float("nan"), device=DEV, dtype=torch.float32)
    sk.csa_index_score(rows, dev(q, qs), dev(w), keysd, scores, m=4, W=128, k=k)
    sk.csa_index_topk(rows, dev(q, qs), dev(w), keysd, out_idx, m=4, W=128, k=k)
    torch.cuda.synchronize()
    gi, gs = host(out_idx), host(scores)
    for t in range(T):
        ev = min(method.entries_visible(t, 4, 128), E_cap)
        s = method.index_scores(q[t], w[t], kv[0, :ev])
        if ev:
            assert_scores_close(gs[t, :ev], s, q[t], w[t], kv[0, :ev], rtol=2e-6, what=f"scores row {t}")
        assert np.all(np.isnan(gs[t, ev:])), f"row {t}: scores written past the {ev} visible entries"
        ok, msg = topk_parity(gi[t], method.topk(s, k), s)
        assert ok, f"row {t} (E_vis={ev}): {msg}"


def test_index_causal_mxfp4_many_stages():
    """Causal rows late in a long sequence over MXFP4 keys: the key tiles pass
    through five LDS stages, and the last stage's copy runs past the end of the
    cache (those lanes re-read its last bytes; nothing past the visible tiles is
    stored)."""
    HI, DI, E_cap, R, pos0, k = 64, 128, 4096, 24, 16000, 256
    print(f"index causal mxfp4 many stages R={R} pos0={pos0} E_cap={E_cap}", flush=True)
    rng = np.random.default_rng(77)
    q = rng_store(rng, (R, HI, DI), "bf16")
    w = rng.normal(0, 1, (R, HI)).astype(np.float32)
    _, _, kv, _, _, keysd = _index_inputs(rng, "mxfp4", HI, DI, 1, E_cap)
    rows = sk.RowSpec.causal(R, pos0=pos0)
    cover = min(method.entries_visible(pos0 + R - 1, 4, 128), E_cap)
    scores = torch.full((R, cover + 3), float("nan"), device=DEV, dtype=torch.float32)
    out_idx = torch.full((R, k), -7, device=DEV, dtype=torch.int32)
    sk.csa_index_score(rows, dev(q, "bf16"), dev(w), keysd, scores, m=4, W=128, k=k)
    sk.csa_index_topk(rows, dev(q, "bf16"), dev(w), keysd, out_idx, m=4, W=128, k=k)
    torch.cuda.synchronize()
    gi, gs = host(out_idx), host(scores)
    for i in range(R):
        t = pos0 + i
        ev = min(method.entries_visible(t, 4, 128), E_cap)
        s = method.index_scores(q[i], w[i], kv[0, :ev])
        assert_scores_close(gs[i, :ev], s, q[i], w[i], kv[0, :ev], rtol=2e-6, what=f"scores row {t}")
        assert np.all(np.isnan(gs[i, ev:])), f"row {t}: scores written past the {ev} visible entries"
        ok, msg = topk_parity(gi[i], method.topk(s, k), s)
        assert ok, f"row {t} (E_vis={ev}): {msg}"


# ---------------------------------------------------------------- attention
ATTEND_CASES = [
    # csa, entries, H, D, E_cap, positions, k, out
    (True, "bf16", 64, 512, 4096, [16511, 300, 50], 1024, "f32"),
    (False, "bf16", 32, 128, 512, [65535, 20000, 130, 0], 0, "f32"),
    (False, "bf16", 64, 512, 1024, [131071, 131070], 0, "f32"),
    (True, "e4m3", 64, 512, 4096, [16511, 9000], 2048, "bf16"),
    (False, "e4m3", 64, 512, 8192, [1048575], 0, "bf16"),
    (True, "f32", 8, 64, 1024, [4095, 600, 10], 64, "f32"),
    (False, "f32", 8, 64, 1024, [4095], 0, "f32"),
    (True, "bf16", 16, 256, 1000, [4127, 2000], 200, "bf16"),
    (True, "bf16", 48, 128, 2048, [8319, 5000, 129], 300, "f32"),      # three 16-head tiles
    (False, "e4m3", 112, 64, 1024, [131071, 70000], 0, "f32"),         # seven 16-head tiles
    (False, "bf16", 16, 64, 16384, [16384 * 128 + 255], 0, "f32"),     # 129 splits: merge threads take 2 (m, l)
]


def _attend_case(csa, ent, H, D, E_cap, positions, k, outs, mag=1.0, seed=None):
    """Runs csa_attend / hca_attend on random decode rows (entries and window rows
    of size mag, queries of size 0.3 / mag, so the logits stay of order one) and
    returns the GPU outputs and log-sum-exps with the oracle's."""
    rng = np.random.default_rng(H * D + E_cap if seed is None else seed)
    B = len(positions)
    qs = "f32" if ent == "f32" else "bf16"
    q = rng_store(rng, (B, H, D), qs, 0.3 / mag)
    if ent == "e4m3":
        st = method.store_entries(rng.normal(0, mag, (B * E_cap, D)), "e4m3")
        ev_vals = st["values"].reshape(B, E_cap, D)
        ent_dev = dev_codes(st["codes"].reshape(B, E_cap, D))
        esc = dev(st["scale"].reshape(B, E_cap))
    else:
        ev_vals = rng_store(rng, (B, E_cap, D), ent, mag).astype(np.float64)
        ent_dev, esc = dev(ev_vals, ent), None
    R_w = 128
    win_vals = {}
    rings = np.zeros((B, R_w, D), np.float32)
    for b, t in enumerate(positions):
        wp = method.window_positions(t, 128)          # only the window tokens are ever read
        win_vals[b] = rng_store(rng, (len(wp), D), qs, mag)
        rings[b][wp % R_w] = win_vals[b]
    idx = None
    idx_np = None
    if csa:
        idx_np = np.full((B, k), -1, np.int64)
        for b, t in enumerate(positions):
            ev = min(method.entries_visible(t, 4, 128), E_cap)
            sel = np.sort(rng.choice(ev, size=min(k, ev), replace=False)) if ev else np.zeros(0, np.int64)
            idx_np[b, :len(sel)] = sel
        idx = dev_i32(idx_np)
    odt = torch.float32 if outs == "f32" else torch.bfloat16
    out = torch.zeros(B, H, D, device=DEV, dtype=odt)
    lse = torch.zeros(B, H, device=DEV, dtype=torch.float32)
    rows = sk.RowSpec.decode(dev_i32(positions), max(positions))
    m = 4 if csa else 128
    tau = 1.0 / math.sqrt(128 if D >= 128 else D)
    args = dict(m=m, W=128, softmax_scale=tau, entry_scale=esc, lse=lse)
    if csa:
        sk.csa_attend(rows, dev(q, qs), ent_dev, idx, dev(rings, qs), out, **args)
    else:
        sk.hca_attend(rows, dev(q, qs), ent_dev, dev(rings, qs), out, **args)
    torch.cuda.synchronize()
    go, gl = host(out), host(lse)
    want = []
    for b, t in enumerate(positions):
        if csa:
            sel = idx_np[b][idx_np[b] >= 0]
            items = np.concatenate([ev_vals[b][sel], win_vals[b]])
        else:
            ev = min(method.entries_visible(t, 128, 128), E_cap)
            items = np.concatenate([ev_vals[b][:ev], win_vals[b]])
        o, lse_o, _ = method.attend(q[b], items, tau)
        want.append((o, lse_o))
    return go, gl, want


@pytest.mark.parametrize("csa,ent,H,D,E_cap,positions,k,outs", ATTEND_CASES)
def test_attend_decode(csa, ent, H, D, E_cap, positions, k, outs):
    print(f"attend decode csa={csa} {ent} H={H} D={D} E_cap={E_cap} pos={positions} k={k} out={outs}", flush=True)
    go, gl, want = _attend_case(csa, ent, H, D, E_cap, positions, k, outs)
    for b, (o, lse_o) in enumerate(want):
        if ent == "f32":
            assert_close(go[b], o, rtol=1e-4, what=f"f32 out row {b}")
        else:
            err = assert_close(go[b], o, atol=2e-2, what=f"out row {b}")
            print(f"  row {b}: max abs err {err:.2e} (max |o| {np.abs(o).max():.2f})")
        np.testing.assert_allclose(gl[b], lse_o, rtol=1e-5, atol=1e-5)


# entries, H, D, magnitude: the register-staged kernel (fp8 entries at D = 512 with
# 64 heads, bf16 entries at other shapes) over values far from 1
MAGNITUDE_CASES = [
    ("e4m3", 64, 512, 1e-4),   # per-entry scales near 1e-6: p * scale far below fp16's normal range
    ("e4m3", 64, 512, 1e7),    # per-entry scales near 1e5: p * scale past fp16's largest value
    ("bf16", 16, 128, 1e5),    # values past fp16's largest value
    ("bf16", 16, 128, 1e-6),   # values in fp16's subnormal range
]


@pytest.mark.parametrize("ent,H,D,mag", MAGNITUDE_CASES)
def test_attend_entry_magnitudes(ent, H, D, mag):
    """Entries and window rows of size mag, queries of size 1 / mag: the output
    follows the oracle normwise to 1e-3 of max |o| (P.V takes probabilities, times
    the fp8 scale, as two bf16 parts over bf16 values, with fp32's exponent range;
    an fp16 operand would lose these cases to underflow or overflow)."""
    print(f"attend magnitudes {ent} H={H} D={D} mag={mag:g}", flush=True)
    go, gl, want = _attend_case(True, ent, H, D, 4096, [16511, 9000], 512, "f32", mag=mag,
                                seed=H * D + int(round(math.log10(mag))) + 50)
    for b, (o, lse_o) in enumerate(want):
        err = assert_close(go[b], o, rtol=1e-3, what=f"out row {b}")
        print(f"  row {b}: max err {err:.2e} (max |o| {np.abs(o).max():.3e})")
        np.testing.assert_allclose(gl[b], lse_o, rtol=1e-4, atol=1e-4)


def test_attend_causal_rows_and_determinism():
    """Prefill-style rows (every position a query) over a whole stream window."""
    rng = np.random.default_rng(9)
    T, H, D, E_cap, k = 600, 64, 512, 150, 32
    q = rng_store(rng, (T, H, D), "bf16", 0.3)
    ent = rng_store(rng, (1, E_cap, D), "bf16").astype(np.float64)
    v = rng_store(rng, (1, T, D), "bf16")
    idx_np = np.full((T, k), -1, np.int64)
    for t in range(T):
        ev = min(method.entries_visible(t, 4, 128), E_cap)
        sel = np.sort(rng.choice(ev, size=min(k, ev), replace=False)) if ev else np.zeros(0, np.int64)
        idx_np[t, :len(sel)] = sel
    rows = sk.RowSpec.causal(T)
    outs = []
    for _ in range(2):
        out = torch.zeros(T, H, D, device=DEV, dtype=torch.float32)
        sk.csa_attend(rows, dev(q, "bf16"), dev(ent, "bf16"), dev_i32(idx_np), dev(v, "bf16"), out, m=4, W=128,
                      softmax_scale=1 / math.sqrt(128))
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    go = host(outs[0])
    for t in list(range(0, 140)) + list(range(140, T, 37)) + [T - 1]:
        sel = idx_np[t][idx_np[t] >= 0]
        items = np.concatenate([ent[0][sel], v[0][method.window_positions(t, 128)]])
        o, _, _ = method.attend(q[t], items, 1 / math.sqrt(128))
        assert_close(go[t], o, atol=2e-2, what=f"row {t}")


@pytest.mark.parametrize("H,D,T,E_cap", [(64, 512, 3000, 32), (32, 128, 2900, 16)])
def test_hca_attend_causal_rows(H, D, T, E_cap):
    """HCA prefill: every position a query over all its visible 128:1 entries plus
    its window (rows before the first entry, rows within it, a capped E_cap)."""
    print(f"hca causal rows H={H} D={D} T={T} E_cap={E_cap}", flush=True)
    rng = np.random.default_rng(H + D + T)
    q = rng_store(rng, (T, H, D), "bf16", 0.3)
    ent = rng_store(rng, (1, E_cap, D), "bf16").astype(np.float64)
    v = rng_store(rng, (1, T, D), "bf16")
    rows = sk.RowSpec.causal(T)
    tau = 1 / math.sqrt(128 if D >= 128 else D)
    outs = []
    for _ in range(2):
        out = torch.zeros(T, H, D, device=DEV, dtype=torch.float32)
        lse = torch.zeros(T, H, device=DEV, dtype=torch.float32)
        sk.hca_attend(rows, dev(q, "bf16"), dev(ent, "bf16"), dev(v, "bf16"), out, m=128, W=128, softmax_scale=tau,
                      lse=lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    go, gl = host(outs[0][0]), host(outs[0][1])
    for t in [0, 1, 127, 128, 255, 256, 257, 383, 384, 1000, 2047, 2176, T - 1]:
        ev = min(method.entries_visible(t, 128, 128), E_cap)
        items = np.concatenate([ent[0][:ev], v[0][method.window_positions(t, 128)]])
        o, lse_o, _ = method.attend(q[t], items, tau)
        assert_close(go[t], o, atol=2e-2, what=f"row {t} (E_vis={ev})")
        np.testing.assert_allclose(gl[t], lse_o, rtol=1e-5, atol=1e-5)


def test_attend_rows_longer_than_a_segment():
    """Causal rows whose item lists (k + window) exceed one block's source segment."""
    rng = np.random.default_rng(10)
    T, H, D, E_cap, k = 520, 64, 512, 1500, 1100
    t0 = 5000                                    # rows are positions t0 .. t0 + T - 1
    q = rng_store(rng, (T, H, D), "bf16", 0.3)
    ent = rng_store(rng, (1, E_cap, D), "bf16").astype(np.float64)
    v = rng_store(rng, (1, t0 + T, D), "bf16")
    idx_np = np.full((T, k), -1, np.int64)
    for r in range(T):
        ev = min(method.entries_visible(t0 + r, 4, 128), E_cap)
        n = min(k - (r % 7) * 50, ev)            # some rows padded with -1
        sel = np.sort(rng.choice(ev, size=n, replace=False))
        idx_np[r, :n] = sel
    rows = sk.RowSpec.causal(T, pos0=t0)
    out = torch.zeros(T, H, D, device=DEV, dtype=torch.float32)
    lse = torch.zeros(T, H, device=DEV, dtype=torch.float32)
    sk.csa_attend(rows, dev(q, "bf16"), dev(ent, "bf16"), dev_i32(idx_np), dev(v, "bf16"), out, m=4, W=128,
                  softmax_scale=1 / math.sqrt(128), lse=lse)
    torch.cuda.synchronize()
    go, gl = host(out), host(lse)
    for r in [0, 1, 6, 77, 300, T - 1]:
        t = t0 + r
        sel = idx_np[r][idx_np[r] >= 0]
        items = np.concatenate([ent[0][sel], v[0][method.window_positions(t, 128)]])
        o, lse_o, _ = method.attend(q[r], items, 1 / math.sqrt(128))
        assert_close(go[r], o, atol=2e-2, what=f"row {r}")
        np.testing.assert_allclose(gl[r], lse_o, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("keys_s", ["e4m3", "mxfp4"])
def test_decode_step_replays_as_hip_graph(keys_s):
    """A decode step (index + top-k with sliced rows, fp8 CSA attention on the
    register-staged kernel, bf16 HCA attention on the copy-staged kernel) captured
    as a HIP graph: every replay, with eager work and synchronizations between
    replays, reproduces the eager results bit for bit.  keys_s: the indexer keys'
    storage (unscaled e4m3 or MXFP4 tiles)."""
    print(f"graph replay of a decode step, {keys_s} indexer keys", flush=True)
    torch.manual_seed(11)
    f8, bf = torch.float8_e4m3fn, torch.bfloat16
    B, E_c, E_h, k, H, D = 2, 40000, 1024, 512, 64, 512
    pos = [160127, 100000]
    rows = sk.RowSpec.decode(dev_i32(pos), max(pos))
    if keys_s == "mxfp4":
        keys = sk.mxfp4_pack(torch.randint(0, 16, (B, E_c, 128), device=DEV, dtype=torch.uint8),
                             torch.randint(120, 134, (B, E_c, 4), device=DEV, dtype=torch.uint8))
    else:
        keys = sk.to_key_tiles(torch.randn(B, E_c, 128, device=DEV).to(f8))
    qI = torch.randn(B, 64, 128, device=DEV).to(bf)
    w = torch.randn(B, 64, device=DEV)
    ent_c = torch.randn(B, E_c, D, device=DEV).to(f8)
    sc_c = torch.rand(B, E_c, device=DEV) + 0.5
    ent_h = torch.randn(B, E_h, D, device=DEV).to(bf)
    win = torch.randn(B, 128, D, device=DEV).to(bf)
    qc = (torch.randn(B, H, D, device=DEV) * 0.3).to(bf)
    qh = (torch.randn(B, H, D, device=DEV) * 0.3).to(bf)
    tau = 1 / math.sqrt(128)

    def outputs():
        return (torch.empty(B, k, device=DEV, dtype=torch.int32), torch.empty(B, H, D, device=DEV, dtype=bf),
                torch.empty(B, H, D, device=DEV, dtype=bf))

    def step(o, ws=(None, None, None)):
        idx, oc, oh = o
        w_i = sk.csa_index_topk(rows, qI, w, keys, idx, m=4, W=128, k=k, workspace=ws[0])
        w_c = sk.csa_attend(rows, qc, ent_c, idx, win, oc, m=4, W=128, softmax_scale=tau, entry_scale=sc_c,
                            workspace=ws[1])
        w_h = sk.hca_attend(rows, qh, ent_h, win, oh, m=128, W=128, softmax_scale=tau, workspace=ws[2])
        return w_i, w_c, w_h

    eager = outputs()
    ws = step(eager)
    torch.cuda.synchronize()
    ref = [t.clone() for t in eager]
    gout = outputs()
    step(gout, ws)                                     # warm the captured path once
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step(gout, ws)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in gout:
            t.zero_()
        step(eager)                                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("indices", "csa out", "hca out"), gout, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
        for a, b in zip(eager, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("E,k", [(32735, 1024), (20000, 512)])
def test_topk_select_one_block_threshold_bins(E, k):
    """Selection from given scores on the one-block path: distinct scores, a group
    of 40 equal scores straddling rank k (the lowest indices of the group are
    kept), all-negative scores, all-equal scores, clustered scores (a few
    first-digit bins hold the whole row), k/2 scores tied at the top, and a short
    row."""
    print(f"topk select one block E={E} k={k}", flush=True)
    rng = np.random.default_rng(E + 3 * k)
    pos = [4 * E + 127] * 6 + [4 * 600 + 128]
    R = len(pos)
    s = rng.normal(0, 3, (R, E)).astype(np.float32)
    order = np.argsort(-s[1], kind="stable")
    s[1, order[k - 20:k + 20]] = s[1, order[k]]              # 40 equal scores across rank k
    s[2] = -np.abs(s[2]) - 1.0                               # all negative
    s[3] = 1.5                                               # all equal: the bin holds the whole row
    s[4] = (1000.0 + rng.normal(0, 1e-3, E)).astype(np.float32)   # clustered: a few first-digit bins
    s[5, order[:k // 2]] = s[5, order[0]]                    # half of k tied at the top score
    rows = sk.RowSpec.decode(dev_i32(pos), max(pos))
    out_idx = torch.full((R, k), -7, device=DEV, dtype=torch.int32)
    out_score = torch.zeros(R, k, device=DEV, dtype=torch.float32)
    qI = torch.zeros(R, 64, 128, device=DEV, dtype=torch.bfloat16)
    w = torch.zeros(R, 64, device=DEV)
    keys = sk.key_tiles_empty(R, (E + 31) // 32 * 32, 128, torch.bfloat16, DEV)
    sk.csa_topk_select(rows, dev(s), out_idx, keys_meta=(qI, w, keys), m=4, W=128, k=k, out_score=out_score)
    torch.cuda.synchronize()
    gi, gs = host(out_idx), host(out_score)
    for r, t in enumerate(pos):
        ev = min(method.entries_visible(t, 4, 128), E)
        ora = method.topk(s[r, :ev], k)
        np.testing.assert_array_equal(gi[r], ora, err_msg=f"row {r}")
        sel = gi[r][gi[r] >= 0]
        np.testing.assert_array_equal(gs[r, :len(sel)], s[r, sel])


@pytest.mark.parametrize("E,k,tie", [(40000, 512, 7.0), (70016, 2048, 6.0)])
def test_topk_select_many_blocks_and_ties(E, k, tie):
    """Selection from given scores on the many-blocks-per-row path (rows longer
    than one block holds): a row of equal scores (its threshold bin holds every
    entry, so the final block streams the row), a row with a third of its entries
    tied at the threshold (k of 40000 keeps the survivors within the final block,
    k of 70016 does not), rows of distinct and of clustered scores, and a short
    row."""
    print(f"topk select many blocks E={E} k={k}", flush=True)
    rng = np.random.default_rng(E + k)
    pos = [4 * E + 127, 4 * E + 127, 4 * E + 127, 4 * E + 127, 4 * 900 + 128]
    R = len(pos)
    s = rng.normal(0, 3, (R, E)).astype(np.float32)
    s[0] = 1.5                                             # all tied
    band = rng.choice(E, size=E // 3, replace=False)       # a third of the row tied near the threshold
    s[1, band] = np.float32(tie)
    s[3] = (1000.0 + rng.normal(0, 1e-3, E)).astype(np.float32)   # clustered: few first-digit bins
    rows = sk.RowSpec.decode(dev_i32(pos), max(pos))
    out_idx = torch.full((R, k), -7, device=DEV, dtype=torch.int32)
    out_score = torch.zeros(R, k, device=DEV, dtype=torch.float32)
    qI = torch.zeros(R, 64, 128, device=DEV, dtype=torch.bfloat16)
    w = torch.zeros(R, 64, device=DEV)
    keys = sk.key_tiles_empty(R, E, 128, torch.bfloat16, DEV)
    sk.csa_topk_select(rows, dev(s), out_idx, keys_meta=(qI, w, keys), m=4, W=128, k=k, out_score=out_score)
    torch.cuda.synchronize()
    gi, gs = host(out_idx), host(out_score)
    for r, t in enumerate(pos):
        ev = min(method.entries_visible(t, 4, 128), E)
        ora = method.topk(s[r, :ev], k)
        np.testing.assert_array_equal(gi[r], ora, err_msg=f"row {r}")
        sel = gi[r][gi[r] >= 0]
        np.testing.assert_array_equal(gs[r, :len(sel)], s[r, sel])
