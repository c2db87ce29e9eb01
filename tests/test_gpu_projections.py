"""GPU parity of the decode projections (layer_queries, layer_streams,
layer_output) against oracle.method.project / absorb_queries / layer_output.

Hidden states, weights and attention outputs are bf16 on both sides; the oracle
runs on the same values in fp64.  Error bounds, element by element:
  * a sum of K products of bf16 values (each exact in fp32) accumulated in fp32
    in any order errs by at most K u sum_k |x_k w_k|; u is taken as 2^-23 (twice
    fp32's unit roundoff) so that the bound holds whatever rounding the matrix
    cores apply inside one instruction;
  * a product fed by an inexact operand adds sum_k |w_k| err_k;
  * a bf16 rounding (to nearest even) adds at most 2^-8 of the magnitude.
Intermediate results the library keeps in its workspace (the fp32 head queries
before absorption, the bf16 heads o_h = W_UV^h o~_h) are checked against the
oracle's own intermediate values with the same bounds.  The absorption of many
rows multiplies the head queries as two bf16 parts (hi = bf16(q), lo =
bf16(q - hi), together within 2^-18 |q|), 2 d_h products per output: its bound,
used for every row count, counts 2 d_h terms and adds 2^-18 of the magnitude."""
import ctypes
import functools

import numpy as np
import pytest
import torch

from oracle import method
from tests.gpu_util import DEV, host
from workloads import configs, gen

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("sequence_compressed_kv_amd")

U32 = 2.0 ** -23
U16 = 2.0 ** -8


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.load()


def bf16(a):
    """float32 values rounded to bf16 (float32 array holding the exact values)."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def up(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV).to(dtype).contiguous()


@functools.lru_cache(maxsize=None)
def weights(name: str, li: int):
    wl = configs.BY_NAME[name]
    return {k: bf16(v) for k, v in gen.layer_weights(wl, li).items() if k != "bpos" and k != "bposI"}


def hidden_rows(R: int, d_model: int, seed: int):
    """Decode rows: N(0, 1) hidden states with every 7th row scaled by 8 (heavy tokens)."""
    x = np.random.default_rng(seed).standard_normal((R, d_model)).astype(np.float32)
    x[::7] *= 8.0
    return bf16(x)


def dot_bound(x, W, K=None):
    """fp32 accumulation bound of x @ W.T (x [R][K], W [N][K])."""
    K = x.shape[1] if K is None else K
    return K * U32 * (np.abs(x) @ np.abs(W).T)


def absorbed_bound(qh, bqh, WUK):
    """Bound of the absorbed queries: the head queries' own bound carried through
    |W_UK|, plus the absorption's (2 d_h fp32 terms of the two-part split, and the
    split's 2^-18)."""
    d_h = WUK.shape[1]
    return np.stack([bqh[:, h, :] @ np.abs(WUK[h]) + (2 * d_h * U32 * 1.01 + 2.0 ** -18) *
                     ((np.abs(qh[:, h, :]) + bqh[:, h, :]) @ np.abs(WUK[h])) for h in range(WUK.shape[0])], axis=1)


def check(g, o, bound, rounded: bool, what: str):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    lim = bound + (U16 * (np.abs(o) + bound) if rounded else 0.0)
    err = np.abs(g - o)
    bad = err > lim
    print(f"{what}: max err {err.max():.3e}, max err/limit {np.max(err / np.maximum(lim, 1e-300)):.3f}", flush=True)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside the bound, first at " \
                          f"{np.argwhere(bad)[0].tolist()}: {g[bad][0]!r} vs {o[bad][0]!r} (limit {lim[bad][0]:.3e})"


# ---------------------------------------------------------------- queries
QUERY_CASES = [
    # workload, layer, R, q dtype
    ("pair_decode_128k_bf16", 0, 32, "bf16"),
    ("pair_decode_128k_bf16", 0, 1, "f32"),
    ("pair_decode_128k_bf16", 0, 64, "bf16"),
    ("pair_decode_128k_bf16", 0, 17, "f32"),
    ("pair_decode_1m_fp8", 1, 1, "bf16"),
    ("csa_decode_4k_f32", 0, 1, "f32"),
    ("csa_decode_4k_f32", 0, 50, "bf16"),
    ("hca_decode_64k_bf16", 0, 4, "bf16"),
]


@pytest.mark.parametrize("name,li,R,qd", QUERY_CASES)
def test_layer_queries_parity(name, li, R, qd):
    print(f"layer_queries {name} layer {li} R={R} q={qd}", flush=True)
    wl = configs.BY_NAME[name]
    L = wl.layers[li]
    w = weights(name, li)
    x = hidden_rows(R, wl.d_model, 11 + R)
    tq = torch.float32 if qd == "f32" else torch.bfloat16
    q = torch.full((R, L.H, L.D), float("nan"), device=DEV, dtype=tq)
    csa = L.kind == "csa"
    qI = torch.full((R, L.H_I, L.D_I), float("nan"), device=DEV, dtype=tq) if csa else None
    hw = torch.full((R, L.H_I), float("nan"), device=DEV) if csa else None
    ws = sk.layer_queries(up(x), up(w["W_q"]), q, W_UK=up(w["W_UK"]) if L.absorbed else None,
                          W_iq=up(w["W_iq"]) if csa else None, qI=qI, W_w=up(w["W_w"]) if csa else None, w=hw)
    torch.cuda.synchronize()
    rounded = qd == "bf16"
    qh = method.project(x, w["W_q"]).reshape(R, L.H, L.d_h)
    bqh = dot_bound(x, w["W_q"]).reshape(R, L.H, L.d_h)
    if L.absorbed:
        # the fp32 head queries the library keeps before absorbing them
        qh_gpu = ws[:R * L.H * L.d_h * 4].view(torch.float32).view(R, L.H, L.d_h)
        check(host(qh_gpu), qh, bqh, False, "q_heads")
        q_ora = method.absorb_queries(qh, w["W_UK"])
        check(host(q), q_ora, absorbed_bound(qh, bqh, w["W_UK"]), rounded, "q (absorbed)")
    else:
        check(host(q), qh, bqh, rounded, "q")
    if csa:
        check(host(qI), method.project(x, w["W_iq"]).reshape(R, L.H_I, L.D_I),
              dot_bound(x, w["W_iq"]).reshape(R, L.H_I, L.D_I), rounded, "qI")
        check(host(hw), method.project(x, w["W_w"]), dot_bound(x, w["W_w"]), False, "w")


@pytest.mark.parametrize("d_h,D,H,R", [(64, 256, 8, 3), (256, 512, 4, 20), (128, 128, 16, 33), (64, 256, 8, 520),
                                     (256, 512, 4, 700)])
def test_layer_queries_absorb_head_dims(d_h, D, H, R):
    """Absorption for the other head widths the library takes (synthetic weights)."""
    print(f"layer_queries absorb d_h={d_h} D={D} H={H} R={R}", flush=True)
    rng = np.random.default_rng(d_h + D)
    dm = 1024
    Wq = bf16(rng.standard_normal((H * d_h, dm)).astype(np.float32) / np.sqrt(dm))
    WUK = bf16(rng.standard_normal((H, d_h, D)).astype(np.float32) / np.sqrt(D))
    x = hidden_rows(R, dm, 5)
    q = torch.full((R, H, D), float("nan"), device=DEV)
    ws = sk.layer_queries(up(x), up(Wq), q, W_UK=up(WUK))
    torch.cuda.synchronize()
    qh = method.project(x, Wq).reshape(R, H, d_h)
    bqh = dot_bound(x, Wq).reshape(R, H, d_h)
    if R >= 512:
        # many rows: the head queries as two bf16 parts [R][H][hi | lo]
        parts = host(ws[:R * H * d_h * 4].view(torch.bfloat16).view(R, H, 2, d_h))
        check(parts[:, :, 0] + parts[:, :, 1], qh, bqh + 2.0 ** -18 * (np.abs(qh) + bqh), False, "q_heads (hi + lo)")
    else:
        check(host(ws[:R * H * d_h * 4].view(torch.float32).view(R, H, d_h)), qh, bqh, False, "q_heads")
    q_ora = method.absorb_queries(qh, WUK)
    check(host(q), q_ora, absorbed_bound(qh, bqh, WUK), False, "q (absorbed)")


# ---------------------------------------------------------------- streams
STREAM_CASES = [
    ("pair_decode_128k_bf16", 0, 32, "bf16"),
    ("pair_decode_128k_bf16", 1, 32, "f32"),
    ("pair_decode_128k_bf16", 0, 3, "f32"),
    ("csa_decode_4k_f32", 0, 1, "f32"),
    ("hca_decode_64k_bf16", 0, 4, "bf16"),
]


@pytest.mark.parametrize("name,li,R,od", STREAM_CASES)
def test_layer_streams_parity(name, li, R, od):
    print(f"layer_streams {name} layer {li} R={R} out={od}", flush=True)
    wl = configs.BY_NAME[name]
    L = wl.layers[li]
    w = weights(name, li)
    x = hidden_rows(R, wl.d_model, 31 + R)
    td = torch.float32 if od == "f32" else torch.bfloat16
    outs = {"v": ("W_c", L.D), "g": ("W_g", L.D)}
    if L.kind == "csa":
        outs.update({"vI": ("W_cI", L.D_I), "gI": ("W_gI", L.D_I)})
    t = {k: torch.full((R, n), float("nan"), device=DEV, dtype=td) for k, (_, n) in outs.items()}
    kw = {}
    for k, (wn, _) in outs.items():
        kw[wn] = up(w[wn])
        kw[k] = t[k]
    sk.layer_streams(up(x), **kw)
    torch.cuda.synchronize()
    for k, (wn, _) in outs.items():
        check(host(t[k]), method.project(x, w[wn]), dot_bound(x, w[wn]), od == "bf16", k)


def test_layer_streams_partial():
    """Only the indexer pair: the other outputs stay untouched."""
    wl = configs.PAIR_DEC_128K_BF16
    w = weights(wl.name, 0)
    x = hidden_rows(5, wl.d_model, 77)
    vI = torch.zeros(5, 128, device=DEV)
    gI = torch.zeros(5, 128, device=DEV)
    sk.layer_streams(up(x), W_cI=up(w["W_cI"]), vI=vI, W_gI=up(w["W_gI"]), gI=gI)
    torch.cuda.synchronize()
    check(host(vI), method.project(x, w["W_cI"]), dot_bound(x, w["W_cI"]), False, "vI")
    check(host(gI), method.project(x, w["W_gI"]), dot_bound(x, w["W_gI"]), False, "gI")


@pytest.mark.parametrize("name,li,R", [("pair_decode_128k_bf16", 0, 32), ("pair_decode_128k_bf16", 1, 32),
                                       ("csa_decode_4k_f32", 0, 1), ("pair_decode_1m_fp8", 0, 1)])
def test_layer_inputs_parity(name, li, R):
    """Queries and streams of the same rows in one launch."""
    print(f"layer_inputs {name} layer {li} R={R}", flush=True)
    wl = configs.BY_NAME[name]
    L = wl.layers[li]
    w = weights(name, li)
    x = hidden_rows(R, wl.d_model, 91 + R)
    csa = L.kind == "csa"
    nan = float("nan")
    q = torch.full((R, L.H, L.D), nan, device=DEV, dtype=torch.bfloat16)
    qI = torch.full((R, L.H_I, L.D_I), nan, device=DEV, dtype=torch.bfloat16) if csa else None
    hw = torch.full((R, L.H_I), nan, device=DEV) if csa else None
    st = {"v": ("W_c", L.D), "g": ("W_g", L.D)}
    if csa:
        st.update({"vI": ("W_cI", L.D_I), "gI": ("W_gI", L.D_I)})
    out = {k: torch.full((R, n), nan, device=DEV, dtype=torch.bfloat16) for k, (_, n) in st.items()}
    kw = {}
    for k, (wn, _) in st.items():
        kw[wn] = up(w[wn])
        kw[k] = out[k]
    sk.layer_inputs(up(x), up(w["W_q"]), q, W_UK=up(w["W_UK"]) if L.absorbed else None,
                    W_iq=up(w["W_iq"]) if csa else None, qI=qI, W_w=up(w["W_w"]) if csa else None, w=hw, **kw)
    torch.cuda.synchronize()
    qh = method.project(x, w["W_q"]).reshape(R, L.H, L.d_h)
    bqh = dot_bound(x, w["W_q"]).reshape(R, L.H, L.d_h)
    if L.absorbed:
        q_ora = method.absorb_queries(qh, w["W_UK"])
        check(host(q), q_ora, absorbed_bound(qh, bqh, w["W_UK"]), True, "q (absorbed)")
    else:
        check(host(q), qh, bqh, True, "q")
    if csa:
        check(host(qI), method.project(x, w["W_iq"]).reshape(R, L.H_I, L.D_I),
              dot_bound(x, w["W_iq"]).reshape(R, L.H_I, L.D_I), True, "qI")
        check(host(hw), method.project(x, w["W_w"]), dot_bound(x, w["W_w"]), False, "w")
    for k, (wn, _) in st.items():
        check(host(out[k]), method.project(x, w[wn]), dot_bound(x, w[wn]), True, k)


# ---------------------------------------------------------------- output
def head_outputs(o, W_UV):
    """o_h = W_UV^h o~_h for every row and head, by the oracle's projection."""
    return np.stack([method.project(o[:, h, :], W_UV[h]) for h in range(W_UV.shape[0])], axis=1)


OUTPUT_CASES = [
    ("pair_decode_128k_bf16", 1, 32, "f32"),
    ("pair_decode_128k_bf16", 0, 32, "bf16"),
    ("pair_decode_128k_bf16", 1, 5, "bf16"),
    ("pair_decode_1m_fp8", 0, 1, "bf16"),
    ("hca_decode_64k_bf16", 0, 4, "f32"),
    ("csa_decode_4k_f32", 0, 1, "f32"),
    ("csa_decode_4k_f32", 0, 64, "bf16"),
]


@pytest.mark.parametrize("name,li,R,yd", OUTPUT_CASES)
def test_layer_output_parity(name, li, R, yd):
    print(f"layer_output {name} layer {li} R={R} y={yd}", flush=True)
    wl = configs.BY_NAME[name]
    L = wl.layers[li]
    w = weights(name, li)
    # attention outputs against the latent: convex mixes of latents, |o| ~ 1
    o = bf16(np.random.default_rng(51 + R).standard_normal((R, L.H, L.D)).astype(np.float32) * 0.5)
    td = torch.float32 if yd == "f32" else torch.bfloat16
    y = torch.full((R, wl.d_model), float("nan"), device=DEV, dtype=td)
    ws = sk.layer_output(up(o), up(w["W_o"]), y, W_UV=up(w["W_UV"]) if L.absorbed else None)
    torch.cuda.synchronize()
    HD = L.H * L.d_h
    Wo = w["W_o"]
    if L.absorbed:
        heads = head_outputs(o, w["W_UV"])                              # o_h = W_UV^h o~_h (fp64)
        b1 = L.D * U32 * np.einsum("hkd,rhd->rhk", np.abs(w["W_UV"]), np.abs(o))
        e1 = b1 + U16 * (np.abs(heads) + b1)                            # rounded to bf16 in the workspace
        heads_gpu = host(ws[:R * HD * 2].view(torch.bfloat16).view(R, L.H, L.d_h))
        check(heads_gpu, heads, b1, True, "heads")
        hflat, eflat = heads.reshape(R, HD), e1.reshape(R, HD)
        bound = eflat @ np.abs(Wo).T + HD * U32 * ((np.abs(hflat) + eflat) @ np.abs(Wo).T)
    else:
        hflat = o.reshape(R, HD)
        bound = dot_bound(hflat, Wo)
    y_ora = np.stack([method.layer_output(o[r], Wo, w["W_UV"] if L.absorbed else None) for r in range(R)])
    check(host(y), y_ora, bound, yd == "bf16", "y")


def test_layer_output_consecutive_calls_reuse_workspace():
    """Two calls in a row through one caller-owned workspace, the second smaller."""
    wl = configs.PAIR_DEC_128K_BF16
    L = wl.layers[1]
    w = weights(wl.name, 1)
    Wo, WUV = up(w["W_o"]), up(w["W_UV"])
    o40 = torch.zeros(40, L.H, L.D, device=DEV, dtype=torch.bfloat16)
    y40 = torch.zeros(40, wl.d_model, device=DEV)
    a = sk.output_args(o40, Wo, y40, W_UV=WUV)
    ws = torch.empty(sk.load().layer_output_workspace_size(ctypes.byref(a)), dtype=torch.uint8, device=DEV)
    for R in (40, 9):
        o = bf16(np.random.default_rng(R).standard_normal((R, L.H, L.D)).astype(np.float32) * 0.5)
        y = torch.full((R, wl.d_model), float("nan"), device=DEV)
        sk.layer_output(up(o), Wo, y, W_UV=WUV, workspace=ws)
        torch.cuda.synchronize()
        heads = head_outputs(o, w["W_UV"])
        y_ora = np.stack([method.layer_output(o[r], w["W_o"], w["W_UV"]) for r in range(R)])
        b1 = L.D * U32 * np.einsum("hkd,rhd->rhk", np.abs(w["W_UV"]), np.abs(o))
        e1 = (b1 + U16 * (np.abs(heads) + b1)).reshape(R, -1)
        bound = e1 @ np.abs(w["W_o"]).T + L.H * L.d_h * U32 * ((np.abs(heads).reshape(R, -1) + e1) @ np.abs(w["W_o"]).T)
        check(host(y), y_ora, bound, False, f"y R={R}")


# ---------------------------------------------------------------- many rows (prefill)
@pytest.mark.parametrize("R", [65, 333, 600])
def test_layer_inputs_many_rows(R):
    """Rows in blocks (64 rows, or 256-row GEMM tiles from 512 rows on) with a ragged
    last block: queries (absorbed, indexer) and streams of the 32K prefill layer's
    shapes."""
    print(f"layer_inputs many rows R={R}", flush=True)
    wl = configs.CSA_PREFILL_32K_BF16
    L = wl.layers[0]
    w = weights(wl.name, 0)
    x = hidden_rows(R, wl.d_model, 7 + R)
    q = torch.full((R, L.H, L.D), float("nan"), device=DEV, dtype=torch.bfloat16)
    qI = torch.full((R, L.H_I, L.D_I), float("nan"), device=DEV, dtype=torch.bfloat16)
    hw = torch.full((R, L.H_I), float("nan"), device=DEV)
    v = torch.full((R, L.D), float("nan"), device=DEV)
    gI = torch.full((R, L.D_I), float("nan"), device=DEV)
    sk.layer_inputs(up(x), up(w["W_q"]), q, W_UK=up(w["W_UK"]), W_iq=up(w["W_iq"]), qI=qI, W_w=up(w["W_w"]), w=hw,
                    W_c=up(w["W_c"]), v=v, W_gI=up(w["W_gI"]), gI=gI)
    torch.cuda.synchronize()
    qh = method.project(x, w["W_q"]).reshape(R, L.H, L.d_h)
    bqh = dot_bound(x, w["W_q"]).reshape(R, L.H, L.d_h)
    q_ora = method.absorb_queries(qh, w["W_UK"])
    check(host(q), q_ora, absorbed_bound(qh, bqh, w["W_UK"]), True, "q (absorbed)")
    check(host(qI), method.project(x, w["W_iq"]).reshape(R, L.H_I, L.D_I),
          dot_bound(x, w["W_iq"]).reshape(R, L.H_I, L.D_I), True, "qI")
    check(host(hw), method.project(x, w["W_w"]), dot_bound(x, w["W_w"]), False, "w")
    check(host(v), method.project(x, w["W_c"]), dot_bound(x, w["W_c"]), False, "v")
    check(host(gI), method.project(x, w["W_gI"]), dot_bound(x, w["W_gI"]), False, "gI")


@pytest.mark.parametrize("R", [130, 700])
def test_layer_output_many_rows(R):
    wl = configs.CSA_PREFILL_32K_BF16
    L = wl.layers[0]
    w = weights(wl.name, 0)
    o = bf16(np.random.default_rng(3).standard_normal((R, L.H, L.D)).astype(np.float32) * 0.5)
    y = torch.full((R, wl.d_model), float("nan"), device=DEV)
    ws = sk.layer_output(up(o), up(w["W_o"]), y, W_UV=up(w["W_UV"]))
    torch.cuda.synchronize()
    heads = head_outputs(o, w["W_UV"])
    b1 = L.D * U32 * np.einsum("hkd,rhd->rhk", np.abs(w["W_UV"]), np.abs(o))
    check(host(ws[:R * L.H * L.d_h * 2].view(torch.bfloat16).view(R, L.H, L.d_h)), heads, b1, True, "heads")
    e1 = (b1 + U16 * (np.abs(heads) + b1)).reshape(R, -1)
    Wo = w["W_o"]
    bound = e1 @ np.abs(Wo).T + L.H * L.d_h * U32 * ((np.abs(heads).reshape(R, -1) + e1) @ np.abs(Wo).T)
    y_ora = np.stack([method.layer_output(o[r], Wo, w["W_UV"]) for r in range(R)])
    check(host(y), y_ora, bound, False, "y")


def test_prefill_streams_full_size_sampled():
    """The 32K prefill layer's four stream products over all 32768 rows in one
    launch; 48 rows (both ends, row-block edges, random) against the oracle."""
    wl = configs.CSA_PREFILL_32K_BF16
    w = weights(wl.name, 0)
    R = wl.N
    x = hidden_rows(R, wl.d_model, 123)
    xd = up(x)
    outs = {k: torch.full((R, n), float("nan"), device=DEV, dtype=torch.bfloat16)
            for k, n in (("v", 512), ("g", 512), ("vI", 128), ("gI", 128))}
    sk.layer_streams(xd, W_c=up(w["W_c"]), v=outs["v"], W_g=up(w["W_g"]), g=outs["g"], W_cI=up(w["W_cI"]),
                     vI=outs["vI"], W_gI=up(w["W_gI"]), gI=outs["gI"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 65, 127, 128, R // 2, R - 65, R - 64, R - 2, R - 1],
                                     rng.integers(0, R, 36)]))
    xs = x[rows]
    for k, wn in (("v", "W_c"), ("g", "W_g"), ("vI", "W_cI"), ("gI", "W_gI")):
        assert torch.isfinite(outs[k].float()).all(), k
        check(host(outs[k][torch.from_numpy(rows).to(DEV)]), method.project(xs, w[wn]), dot_bound(xs, w[wn]), True, k)


@pytest.mark.parametrize("R", [1, 3, 40])
def test_projections_smallest_shapes(R):
    """d_model = 128 (one k-step per wave, four-wave blocks) and a 128-dim latent
    with W_UV over 128: the smallest reduction lengths the library takes."""
    rng = np.random.default_rng(R)
    dm, H, d_h, D = 128, 2, 64, 128
    Wq = bf16(rng.standard_normal((H * d_h, dm)).astype(np.float32) / np.sqrt(dm))
    WUK = bf16(rng.standard_normal((H, d_h, D)).astype(np.float32) / np.sqrt(D))
    Wc = bf16(rng.standard_normal((D, dm)).astype(np.float32) / np.sqrt(dm))
    WUV = bf16(rng.standard_normal((H, d_h, D)).astype(np.float32) / np.sqrt(D))
    Wo = bf16(rng.standard_normal((dm, H * d_h)).astype(np.float32) / np.sqrt(H * d_h))
    x = hidden_rows(R, dm, 9)
    q = torch.full((R, H, D), float("nan"), device=DEV)
    v = torch.full((R, D), float("nan"), device=DEV)
    sk.layer_inputs(up(x), up(Wq), q, W_UK=up(WUK), W_c=up(Wc), v=v)
    torch.cuda.synchronize()
    qh = method.project(x, Wq).reshape(R, H, d_h)
    bqh = dot_bound(x, Wq).reshape(R, H, d_h)
    check(host(q), method.absorb_queries(qh, WUK), absorbed_bound(qh, bqh, WUK), False, "q")
    check(host(v), method.project(x, Wc), dot_bound(x, Wc), False, "v")
    o = bf16(rng.standard_normal((R, H, D)).astype(np.float32) * 0.5)
    y = torch.full((R, dm), float("nan"), device=DEV)
    sk.layer_output(up(o), up(Wo), y, W_UV=up(WUV))
    torch.cuda.synchronize()
    heads = head_outputs(o, WUV)
    b1 = D * U32 * np.einsum("hkd,rhd->rhk", np.abs(WUV), np.abs(o))
    e1 = (b1 + U16 * (np.abs(heads) + b1)).reshape(R, -1)
    bound = e1 @ np.abs(Wo).T + H * d_h * U32 * ((np.abs(heads).reshape(R, -1) + e1) @ np.abs(Wo).T)
    y_ora = np.stack([method.layer_output(o[r], Wo, WUV) for r in range(R)])
    check(host(y), y_ora, bound, False, "y")
