"""Parity at the five workloads' full sizes, in the launch configuration of the
timed step.

Each test
  1. builds the workload's caches with the library's compressors;
  2. checks the stored caches of sampled sequences against the oracle in code
     space (equal codes, or a rounding flip explained by the fp32 error of the
     pooled sum);
  3. overwrites those sequences' indexer keys and entries with the oracle's
     stored values, so that both sides rank and attend identical caches (a
     legitimate one-ulp flip in a key could otherwise move a top-k boundary);
  4. runs the step exactly as it is timed and compares the sampled rows' top-k
     (exact, up to swaps of near-equal oracle scores) and outputs with the oracle.

Inputs: the host recipe (workloads.gen) for the small CSA workload; elsewhere
seeded GPU-drawn streams and queries (workloads.gen.gpu_*), copied back to the
host for the oracle.
"""
import math

import numpy as np
import pytest
import torch

from oracle import method
from tests.compare import assert_close, bf16_code_flips, blocked_compress, e4m3_flips, mxfp4_flips, topk_parity
from tests.gpu_util import DEV, dev, dev_codes, dev_i32, host
from workloads import (CSA_DEC_4K_F32, CSA_PREFILL_32K_BF16, HCA_DEC_64K_BF16, PAIR_DEC_1M_FP8,
                       PAIR_DEC_128K_BF16, gen)

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("sequence_compressed_kv_amd")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.load()


# ---------------------------------------------------------------- oracle side
def f32(t):
    return t.float().cpu().numpy()


def oracle_pool(v, g, bpos, m, o, store, keys=False):
    """Oracle entries (or keys) of one sequence: unrounded, magnitude of the fp32
    error scale (the same pool over |v|) and the stored form."""
    c = blocked_compress(v, g, bpos, m, o)
    mag = blocked_compress(np.abs(v), g, bpos, m, o)
    st = method.store_keys(c, store) if keys else method.store_entries(c, store)
    return c, mag, st


def check_codes(what, store, got, c, mag, st, got_scale=None, keys=False):
    """Stored GPU values of one sequence vs the oracle's, in code space."""
    E = c.shape[0]
    if store == "f32":
        assert_close(host(got)[:E], c, rtol=1e-5, what=what)
    elif store == "bf16":
        n_bad, n_unexp = bf16_code_flips(host(got)[:E], c, st["values"], magnitude=mag)
        assert n_unexp == 0, f"{what}: {n_unexp} of {n_bad} bf16 codes differ"
    else:
        gc = host(got)[:E]
        if not keys:
            np.testing.assert_allclose(got_scale.cpu().numpy()[:E].astype(np.float64), st["scale"], rtol=2e-6)
            y, ymag = c / st["scale"][:, None], mag / st["scale"][:, None]
        else:
            y, ymag = c, mag
        n_bad, n_unexp = e4m3_flips(gc, st["codes"], y, ymag)
        assert n_unexp == 0, f"{what}: {n_unexp} of {n_bad} e4m3 codes differ"


def upload_store(st, store, like):
    if store == "e4m3":
        return dev_codes(st["codes"])
    return dev(st["values"], store).to(like.dtype)


def tau_of(L):
    return 1.0 / math.sqrt(L.d_h)


# sequences of the batch-32 step compared in full: one for each residue modulo 8 (the
# attention kernel deals a row's blocks to the XCD of that residue), spread over the batch
SEQ_SAMPLE = [0, 9, 18, 27, 4, 13, 22, 31]


# ---------------------------------------------------------------- small CSA decode, fp32 (host recipe)
def test_csa_decode_4k_f32():
    wl = CSA_DEC_4K_F32
    L = wl.layers[0]
    print(f"{wl.name}: B={wl.B} N={wl.N}", flush=True)
    inp = gen.decode_inputs(wl, 0)
    st, q, w = inp["layers"][0]["streams"], inp["layers"][0]["queries"], inp["layers"][0]["weights"]
    t = inp["t"]
    E = wl.N // L.m
    ent = torch.zeros(1, E, L.D, device=DEV)
    keys = sk.key_tiles_empty(1, E, L.D_I, torch.float32, DEV)
    sk.csa_compress(sk.Pool(dev(st["v"])[None], dev(st["g"])[None], dev(w["bpos"]), ent),
                    sk.Pool(dev(st["vI"])[None], dev(st["gI"])[None], dev(w["bposI"]), keys,
                            layout=sk.LAYOUT_KEY_TILES), m=L.m, o=L.o)
    torch.cuda.synchronize()
    c, mag, se = oracle_pool(st["v"], st["g"], w["bpos"], L.m, L.o, "f32")
    cI, magI, sI = oracle_pool(st["vI"], st["gI"], w["bposI"], L.m, L.o, "f32", keys=True)
    check_codes("entries", "f32", ent[0], c, mag, se)
    check_codes("keys", "f32", sk.from_key_tiles(keys)[0], cI, magI, sI, keys=True)
    ent[0] = dev(se["values"])
    keys.copy_(sk.to_key_tiles(dev(sI["values"])[None]))
    rows = sk.RowSpec.decode(dev_i32([t]), t)
    idx = torch.zeros(1, L.k, dtype=torch.int32, device=DEV)
    sk.csa_index_topk(rows, dev(q["qI"]), dev(q["w"]), keys, idx, m=L.m, W=L.W, k=L.k)
    out = torch.zeros(1, L.H, L.D, device=DEV)
    lse = torch.zeros(1, L.H, device=DEV)
    sk.csa_attend(rows, dev(q["q"]), ent, idx, dev(st["v"])[None], out, m=L.m, W=L.W,
                  softmax_scale=tau_of(L), lse=lse)
    torch.cuda.synchronize()
    r = method.csa_row(t, q["q"][0], q["qI"][0], q["w"][0], se["values"], sI["values"], st["v"], L.m, L.W, L.k,
                       tau_of(L))
    ok, msg = topk_parity(host(idx)[0], r["idx"], r["scores"])
    assert ok, msg
    assert_close(host(out)[0], r["o"], rtol=1e-4, what="CSA output")
    np.testing.assert_allclose(host(lse)[0], r["lse"], rtol=1e-5)


# ---------------------------------------------------------------- HCA decode, bf16, batch 4 at 64K
def test_hca_decode_64k_bf16():
    wl = HCA_DEC_64K_BF16
    L = wl.layers[0]
    print(f"{wl.name}: B={wl.B} N={wl.N}", flush=True)
    weights = gen.gpu_weights(wl, DEV)
    w0 = weights[0]
    E = wl.N // L.m
    bf = torch.bfloat16
    ent = torch.empty(wl.B, E, L.D, device=DEV, dtype=bf)
    win = torch.empty(wl.B, L.W, L.D, device=DEV, dtype=bf)
    slots = torch.arange(wl.N - L.W, wl.N, device=DEV) % L.W
    host_v = []
    for b in range(wl.B):
        s = gen.gpu_sequence_streams(wl, b, weights, DEV)[0]
        sk.hca_compress(sk.Pool(s["v"][None], s["g"][None], w0["bpos"].contiguous(), ent[b:b + 1]), m=L.m, o=L.o)
        win[b, slots] = s["v"][wl.N - L.W:]
        torch.cuda.synchronize()
        v, g = f32(s["v"]), f32(s["g"])
        c, mag, se = oracle_pool(v, g, f32(w0["bpos"]), L.m, L.o, "bf16")
        check_codes(f"entries seq {b}", "bf16", ent[b], c, mag, se)
        ent[b] = upload_store(se, "bf16", ent)
        host_v.append((v, se["values"]))
    q = gen.gpu_queries(wl, 0, wl.B, DEV)["q"]
    t = wl.N - 1
    rows = sk.RowSpec.decode(torch.full((wl.B,), t, dtype=torch.int32, device=DEV), t)
    out = torch.zeros(wl.B, L.H, L.D, device=DEV)
    lse = torch.zeros(wl.B, L.H, device=DEV)
    sk.hca_attend(rows, q, ent, win, out, m=L.m, W=L.W, softmax_scale=tau_of(L), lse=lse)
    torch.cuda.synchronize()
    for b in range(wl.B):
        v, vals = host_v[b]
        r = method.hca_row(t, f32(q[b]), vals, v, L.m, L.W, tau_of(L))
        err = assert_close(host(out)[b], r["o"], atol=2e-2, what=f"HCA output seq {b}")
        print(f"  seq {b}: max abs err {err:.2e}", flush=True)
        np.testing.assert_allclose(host(lse)[b], r["lse"], rtol=1e-5, atol=1e-5)


# ---------------------------------------------------------------- CSA prefill, bf16, 32K causal rows
def test_csa_prefill_32k_bf16():
    wl = CSA_PREFILL_32K_BF16
    L = wl.layers[0]
    T = wl.N
    print(f"{wl.name}: T={T}", flush=True)
    weights, st, qs = gen.gpu_prefill_inputs(wl, DEV)
    w0 = weights[0]
    E = T // L.m
    bf = torch.bfloat16
    ent = torch.empty(1, E, L.D, device=DEV, dtype=bf)
    keys = sk.key_tiles_empty(1, E, L.D_I, bf, DEV)
    sk.csa_compress(sk.Pool(st["v"][None], st["g"][None], w0["bpos"].contiguous(), ent),
                    sk.Pool(st["vI"][None], st["gI"][None], w0["bposI"].contiguous(), keys,
                            layout=sk.LAYOUT_KEY_TILES), m=L.m, o=L.o)
    torch.cuda.synchronize()
    v = f32(st["v"])
    c, mag, se = oracle_pool(v, f32(st["g"]), f32(w0["bpos"]), L.m, L.o, "bf16")
    cI, magI, sI = oracle_pool(f32(st["vI"]), f32(st["gI"]), f32(w0["bposI"]), L.m, L.o, "bf16", keys=True)
    check_codes("entries", "bf16", ent[0], c, mag, se)
    check_codes("keys", "bf16", sk.from_key_tiles(keys)[0], cI, magI, sI, keys=True)
    ent[0] = upload_store(se, "bf16", ent)
    keys.copy_(sk.to_key_tiles(dev(sI["values"], "bf16")[None]))
    rows = sk.RowSpec.causal(T)
    idx = torch.empty(T, L.k, dtype=torch.int32, device=DEV)
    sk.csa_index_topk(rows, qs["qI"], qs["w"], keys, idx, m=L.m, W=L.W, k=L.k)
    out = torch.empty(T, L.H, L.D, device=DEV)
    sk.csa_attend(rows, qs["q"], ent, idx, st["v"][None], out, m=L.m, W=L.W, softmax_scale=tau_of(L))
    torch.cuda.synchronize()
    heavy = gen.heavy_positions(wl, 0)
    # rows compared: every 16th; edge rows; a full block of 8 consecutive rows (the
    # causal scoring kernel's unit) around every boundary of its 256-key LDS stages
    # (visible count 256 s: position 1024 s + 128); each heavy token and the two
    # rows after it (queries whose window holds it)
    edges = {0, 1, 127, 128, 131, 132, 133, 200, 1000, 2179, 2180, 2500, T - 2, T - 1}
    blocks = {8 * ((1024 * s_ + 128) // 8) + i for s_ in range(T // 1024) for i in range(-8, 8)}
    near_heavy = {int(h) + d for h in heavy for d in (0, 1, 2)}
    sample = sorted(x for x in set(range(0, T, 16)) | edges | blocks | near_heavy if 0 <= x < T)
    print(f"  comparing {len(sample)} of {T} rows", flush=True)
    gi = host(idx)
    sel = torch.tensor(sample, device=DEV)
    go = host(out[sel])
    tau = tau_of(L)
    qh, qIh, wh = f32(qs["q"][sel]), f32(qs["qI"][sel]), qs["w"][sel].cpu().numpy()
    worst = 0.0
    for i, t in enumerate(sample):
        r = method.csa_row(t, qh[i], qIh[i], wh[i], se["values"], sI["values"], v, L.m, L.W, L.k, tau)
        ok, msg = topk_parity(gi[t], r["idx"], r["scores"])
        assert ok, f"row {t} (E_vis={r['e_vis']}): {msg}"
        err = assert_close(go[i], r["o"], atol=2e-2, what=f"row {t}")
        worst = max(worst, err)
    print(f"  {len(sample)} rows: top-k match, max abs err {worst:.2e}", flush=True)


# ---------------------------------------------------------------- CSA+HCA pair decode, bf16, batch 32 at 128K
def test_pair_decode_128k_bf16():
    """The timed workload: caches built by the timed step's builder, the step's four calls."""
    import bench
    wl = PAIR_DEC_128K_BF16
    csa, hca = wl.layers
    B, t = wl.B, wl.N - 1
    print(f"{wl.name}: B={B} N={wl.N}", flush=True)
    c, h = bench.build_caches(wl, DEV, sk, torch, gen)
    weights = gen.gpu_weights(wl, DEV)
    qc = gen.gpu_queries(wl, 0, B, DEV)
    qh = gen.gpu_queries(wl, 1, B, DEV)
    sampled = SEQ_SAMPLE
    tau = tau_of(csa)
    ora = {}
    for b in sampled:
        s_c, s_h = gen.gpu_sequence_streams(wl, b, weights, DEV)
        vc, vh = f32(s_c["v"]), f32(s_h["v"])
        cc, magc, sc = oracle_pool(vc, f32(s_c["g"]), f32(weights[0]["bpos"]), csa.m, csa.o, "bf16")
        cI, magI, sI = oracle_pool(f32(s_c["vI"]), f32(s_c["gI"]), f32(weights[0]["bposI"]), csa.m, csa.o, "bf16",
                                   keys=True)
        ch, magh, sh = oracle_pool(vh, f32(s_h["g"]), f32(weights[1]["bpos"]), hca.m, hca.o, "bf16")
        del s_c, s_h
        check_codes(f"CSA entries seq {b}", "bf16", c["entries"][b], cc, magc, sc)
        check_codes(f"CSA keys seq {b}", "bf16", sk.from_key_tiles(c["keys"][b:b + 1])[0], cI, magI, sI, keys=True)
        check_codes(f"HCA entries seq {b}", "bf16", h["entries"][b], ch, magh, sh)
        c["entries"][b] = upload_store(sc, "bf16", c["entries"])
        c["keys"][b:b + 1] = sk.to_key_tiles(dev(sI["values"], "bf16")[None])
        h["entries"][b] = upload_store(sh, "bf16", h["entries"])
        # the oracle's rows now (they need only host data), keeping the big arrays short-lived
        r = method.csa_row(t, f32(qc["q"][b]), f32(qc["qI"][b]), qc["w"][b].cpu().numpy(), sc["values"],
                           sI["values"], vc, csa.m, csa.W, csa.k, tau)
        rh = method.hca_row(t, f32(qh["q"][b]), sh["values"], vh, hca.m, hca.W, tau)
        ora[b] = (r["idx"], r["scores"], r["o"], rh["o"])
        del vc, vh, cc, magc, sc, cI, magI, sI, ch, magh, sh, r, rh
    rows = sk.RowSpec.decode(torch.full((B,), t, dtype=torch.int32, device=DEV), t)
    idx = torch.empty(B, csa.k, dtype=torch.int32, device=DEV)
    out_c = torch.empty(B, csa.H, csa.D, device=DEV)
    out_h = torch.empty(B, hca.H, hca.D, device=DEV)
    sk.csa_index_topk(rows, qc["qI"], qc["w"], c["keys"], idx, m=csa.m, W=csa.W, k=csa.k)
    sk.csa_attend(rows, qc["q"], c["entries"], idx, c["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau)
    sk.hca_attend(rows, qh["q"], h["entries"], h["win"], out_h, m=hca.m, W=hca.W, softmax_scale=tau)
    torch.cuda.synchronize()
    gi = host(idx)
    for b in sampled:
        r_idx, r_scores, r_o, rh_o = ora[b]
        ok, msg = topk_parity(gi[b], r_idx, r_scores)
        assert ok, f"seq {b}: {msg}"
        ec = assert_close(host(out_c[b]), r_o, atol=2e-2, what=f"CSA output seq {b}")
        eh = assert_close(host(out_h[b]), rh_o, atol=2e-2, what=f"HCA output seq {b}")
        print(f"  seq {b}: CSA max abs err {ec:.2e}, HCA {eh:.2e}", flush=True)


# ---------------------------------------------------------------- the same step with MXFP4 indexer keys
def test_pair_decode_128k_mxfp4_keys():
    """The 128K batch-32 step with the indexer keys pooled into MXFP4 tiles by the
    timed step's builder: stored blocks against the oracle's (scales and codes, flips
    only where the fp32 pooling error explains them), then the step's top-k and CSA
    output against the oracle on the oracle's keys."""
    import bench
    wl = PAIR_DEC_128K_BF16
    csa, hca = wl.layers
    B, t = wl.B, wl.N - 1
    print(f"{wl.name} with MXFP4 indexer keys: B={B} N={wl.N}", flush=True)
    c, h = bench.build_caches(wl, DEV, sk, torch, gen, fp4_keys=True)
    keys = c["keys_fp4"]
    weights = gen.gpu_weights(wl, DEV)
    qc = gen.gpu_queries(wl, 0, B, DEV)
    sampled = SEQ_SAMPLE
    tau = tau_of(csa)
    ora = {}
    codes_all, scale_all = sk.mxfp4_unpack(keys)
    for b in sampled:
        s_c, _ = gen.gpu_sequence_streams(wl, b, weights, DEV)
        vc = f32(s_c["v"])
        cI = blocked_compress(f32(s_c["vI"]), f32(s_c["gI"]), f32(weights[0]["bposI"]), csa.m, csa.o)
        magI = blocked_compress(np.abs(f32(s_c["vI"])), f32(s_c["gI"]), f32(weights[0]["bposI"]), csa.m, csa.o)
        del s_c
        E = cI.shape[0]
        n_diff, n_un = mxfp4_flips(codes_all[b, :E].cpu().numpy(), scale_all[b, :E].cpu().numpy(), cI, magI)
        assert n_un == 0, f"seq {b}: {n_un} of {n_diff} MXFP4 scales/codes unexplained"
        print(f"  seq {b}: {n_diff} MXFP4 flips explained by the fp32 pooling error", flush=True)
        st = method.store_keys(cI, "mxfp4")
        keys.tiles[b:b + 1] = sk.mxfp4_pack(torch.from_numpy(st["codes"])[None],
                                            torch.from_numpy(st["scale"])[None]).tiles.to(DEV)
        ent = c["entries"][b].float().cpu().numpy().astype(np.float64)
        r = method.csa_row(t, f32(qc["q"][b]), f32(qc["qI"][b]), qc["w"][b].cpu().numpy(), ent, st["values"], vc,
                           csa.m, csa.W, csa.k, tau)
        ora[b] = (r["idx"], r["scores"], r["o"])
        del vc, cI, magI, ent, r
    rows = sk.RowSpec.decode(torch.full((B,), t, dtype=torch.int32, device=DEV), t)
    idx = torch.empty(B, csa.k, dtype=torch.int32, device=DEV)
    out_c = torch.empty(B, csa.H, csa.D, device=DEV)
    sk.csa_index_topk(rows, qc["qI"], qc["w"], keys, idx, m=csa.m, W=csa.W, k=csa.k)
    sk.csa_attend(rows, qc["q"], c["entries"], idx, c["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau)
    torch.cuda.synchronize()
    gi = host(idx)
    for b in sampled:
        r_idx, r_scores, r_o = ora[b]
        ok, msg = topk_parity(gi[b], r_idx, r_scores)
        assert ok, f"seq {b}: {msg}"
        ec = assert_close(host(out_c[b]), r_o, atol=2e-2, what=f"CSA output seq {b}")
        print(f"  seq {b}: top-k matches, CSA max abs err {ec:.2e}", flush=True)


# ---------------------------------------------------------------- CSA+HCA pair decode at 1M, fp8 caches
@pytest.mark.slow
@pytest.mark.parametrize("keys_s", ["e4m3", "mxfp4"])
def test_pair_decode_1m_fp8(keys_s):
    """keys_s: the indexer keys' storage, unscaled e4m3 or MXFP4 (FP4 blocks of 32
    channels with a power-of-two scale: the pages' FP4 indexer at 1M context)."""
    wl = PAIR_DEC_1M_FP8
    csa, hca = wl.layers
    t = wl.N - 1
    print(f"{wl.name}: B={wl.B} N={wl.N} indexer keys {keys_s}", flush=True)
    weights = gen.gpu_weights(wl, DEV)
    Ec, Eh = wl.N // csa.m, wl.N // hca.m
    f8, bf = torch.float8_e4m3fn, torch.bfloat16
    ent_c = torch.empty(1, Ec, csa.D, device=DEV, dtype=torch.uint8).view(f8)
    sc_c = torch.empty(1, Ec, device=DEV)
    keys = (sk.Mxfp4Keys.empty(1, Ec, csa.D_I, DEV) if keys_s == "mxfp4"
            else sk.key_tiles_empty(1, Ec, csa.D_I, torch.uint8, DEV).view(f8))
    ent_h = torch.empty(1, Eh, hca.D, device=DEV, dtype=torch.uint8).view(f8)
    sc_h = torch.empty(1, Eh, device=DEV)
    win_c = torch.empty(1, csa.W, csa.D, device=DEV, dtype=bf)
    win_h = torch.empty(1, hca.W, hca.D, device=DEV, dtype=bf)
    s_c, s_h = gen.gpu_sequence_streams(wl, 0, weights, DEV)
    sk.csa_compress(sk.Pool(s_c["v"][None], s_c["g"][None], weights[0]["bpos"].contiguous(), ent_c, sc_c),
                    sk.Pool(s_c["vI"][None], s_c["gI"][None], weights[0]["bposI"].contiguous(), keys,
                            layout=sk.LAYOUT_KEY_TILES), m=csa.m, o=csa.o)
    sk.hca_compress(sk.Pool(s_h["v"][None], s_h["g"][None], weights[1]["bpos"].contiguous(), ent_h, sc_h),
                    m=hca.m, o=hca.o)
    slots = torch.arange(wl.N - csa.W, wl.N, device=DEV) % csa.W
    win_c[0, slots] = s_c["v"][wl.N - csa.W:]
    win_h[0, slots] = s_h["v"][wl.N - hca.W:]
    torch.cuda.synchronize()
    vc, vh = f32(s_c["v"]), f32(s_h["v"])
    cc, magc, stc = oracle_pool(vc, f32(s_c["g"]), f32(weights[0]["bpos"]), csa.m, csa.o, "e4m3")
    cI, magI, stI = oracle_pool(f32(s_c["vI"]), f32(s_c["gI"]), f32(weights[0]["bposI"]), csa.m, csa.o, keys_s,
                                keys=True)
    ch, magh, sth = oracle_pool(vh, f32(s_h["g"]), f32(weights[1]["bpos"]), hca.m, hca.o, "e4m3")
    del s_c, s_h
    check_codes("CSA entries", "e4m3", ent_c[0], cc, magc, stc, got_scale=sc_c[0])
    if keys_s == "mxfp4":
        gcodes, gscale = (x[0, :Ec].cpu().numpy() for x in sk.mxfp4_unpack(keys))
        n_diff, n_un = mxfp4_flips(gcodes, gscale, cI, magI)
        assert n_un == 0, f"CSA keys: {n_un} of {n_diff} MXFP4 scales/codes unexplained"
    else:
        check_codes("CSA keys", "e4m3", sk.from_key_tiles(keys)[0], cI, magI, stI, keys=True)
    check_codes("HCA entries", "e4m3", ent_h[0], ch, magh, sth, got_scale=sc_h[0])
    del cc, magc, cI, magI, ch, magh
    ent_c[0] = dev_codes(stc["codes"])
    sc_c[0] = dev(stc["scale"])
    if keys_s == "mxfp4":
        keys.tiles.copy_(sk.mxfp4_pack(torch.from_numpy(stI["codes"])[None],
                                       torch.from_numpy(stI["scale"])[None]).tiles.to(DEV))
    else:
        keys.copy_(sk.to_key_tiles(dev_codes(stI["codes"])[None]))
    ent_h[0] = dev_codes(sth["codes"])
    sc_h[0] = dev(sth["scale"])
    qc = gen.gpu_queries(wl, 0, 1, DEV)
    qh = gen.gpu_queries(wl, 1, 1, DEV)
    rows = sk.RowSpec.decode(dev_i32([t]), t)
    idx = torch.empty(1, csa.k, dtype=torch.int32, device=DEV)
    out_c = torch.empty(1, csa.H, csa.D, device=DEV, dtype=bf)
    out_h = torch.empty(1, hca.H, hca.D, device=DEV, dtype=bf)
    tau = tau_of(csa)
    sk.csa_index_topk(rows, qc["qI"], qc["w"], keys, idx, m=csa.m, W=csa.W, k=csa.k)
    sk.csa_attend(rows, qc["q"], ent_c, idx, win_c, out_c, m=csa.m, W=csa.W, softmax_scale=tau, entry_scale=sc_c)
    sk.hca_attend(rows, qh["q"], ent_h, win_h, out_h, m=hca.m, W=hca.W, softmax_scale=tau, entry_scale=sc_h)
    torch.cuda.synchronize()
    r = method.csa_row(t, f32(qc["q"][0]), f32(qc["qI"][0]), qc["w"][0].cpu().numpy(), stc["values"],
                       stI["values"], vc, csa.m, csa.W, csa.k, tau)
    ok, msg = topk_parity(host(idx)[0], r["idx"], r["scores"])
    assert ok, msg
    ec = assert_close(host(out_c)[0], r["o"], atol=2e-2, what="CSA output")
    rh = method.hca_row(t, f32(qh["q"][0]), sth["values"], vh, hca.m, hca.W, tau)
    eh = assert_close(host(out_h)[0], rh["o"], atol=2e-2, what="HCA output")
    print(f"  CSA max abs err {ec:.2e}, HCA {eh:.2e}", flush=True)
