"""Plain fp64 CPU definition of the CSA / HCA compressed-attention hot path.

TEST INFRASTRUCTURE ONLY (see the package header).

Sources.  The pages describe the method in words; where they leave a formula
open, the CSA decode workload definition (fp32, one query at t = 4095 over a
4096-token prefix) fixes it, and the other workloads generalise it:

* Compressor (knightli.com DeepSeek-V4 KV-cache article, "CSA: compresion 4x
  mas recuperacion dispersa": a learned pool over overlapping windows, about
  four tokens per entry; "HCA: compresion 128x mas atencion densa": 128 tokens
  per entry; bayesiansapien.github.io "DeepSeek-V4: interleaved compressed
  attention ...", TL;DR: a learned token compressor).  The workload definition
  fixes it as: entry j pools tokens [m j - o, m j + m); per channel d the gate
  logits g_i[d] + Bpos[i - m j + o][d] are softmaxed over the window and weight
  the values v_i[d].
* Lightning indexer and top-k (same article, CSA section: the indexer scores
  the compressed blocks and the top-k are kept; kongchang.com "DeepSeek V4 Deep
  Dive", "Innovation 1: Hybrid Attention Architecture").  Fixed as
  s_j = sum_h w_h * ReLU(qI_h . kI_j); ties go to the lower entry index.
* Visibility: entry j is usable by query t iff m (j + 1) <= t - W.
* Attention (same article, "Ventana deslizante": compressed branches are
  concatenated with the sliding-window K/V): one softmax over the selected (CSA)
  or all visible (HCA) entries together with the raw tokens [t - W + 1, t].
* Shared latent K = V of width D with queries absorbed into it when D exceeds
  the head dim (the same article, "Varias generaciones de optimizacion de KV
  Cache", MLA: the per-token KV is a compressed latent vector).

Every function is written from these statements, not from any listing.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import codecs


# ---------------------------------------------------------------- visibility and window
def entries_visible(t: int, m: int, W: int) -> int:
    """Count of entries query t may use: entry j is visible iff m*(j+1) <= t - W."""
    return max(0, (t - W) // m)


def window_positions(t: int, W: int) -> np.ndarray:
    """Raw tokens in the sliding window of query t: [max(0, t-W+1), t] (t included)."""
    return np.arange(max(0, t - W + 1), t + 1)


# ---------------------------------------------------------------- compressor
def compress(v, g, bpos, m: int, o: int, chunk: Optional[int] = None) -> np.ndarray:
    """Gated per-channel softmax pool of one sequence.

    v, g : [N][D] values and gate logits per token; bpos : [m+o][D] position bias.
    Returns c : [N // m][D] fp64, one row per complete entry j (tokens up to m j + m - 1).
    Window tokens before position 0 do not exist and take no part in the softmax.
    """
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    bpos = np.asarray(bpos, np.float64)
    N, D = v.shape
    L = m + o
    assert bpos.shape == (L, D)
    E = N // m
    out = np.empty((E, D))
    if chunk is None:                       # bound the [entries][window][D] temporaries
        chunk = max(1, (1 << 22) // (L * D))
    for j0 in range(0, E, chunk):
        j = np.arange(j0, min(E, j0 + chunk))
        tok = m * j[:, None] - o + np.arange(L)[None, :]          # [J][L]; window slot l = i - m j + o
        valid = tok >= 0
        tok_c = np.where(valid, tok, 0)
        logits = g[tok_c] + bpos[None, :, :]                      # [J][L][D]
        logits = np.where(valid[:, :, None], logits, -np.inf)
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        out[j] = (p * v[tok_c]).sum(axis=1)
    return out


def store_entries(c, store: str) -> Dict[str, Optional[np.ndarray]]:
    """Round compressed entries to their storage format.

    f32/bf16: RNE.  e4m3: per-entry scale = fp32(max_d |c_j[d]| / 448) (1 if the
    row is zero); codes = saturating RNE of c / scale; the stored value is
    code * scale.  Returns dict(values=fp64 dequantised, codes=uint8|None,
    scale=fp64 (fp32-valued)|None).
    """
    c = np.asarray(c, np.float64)
    if store == "f32":
        return {"values": codecs.round_f32(c), "codes": None, "scale": None}
    if store == "bf16":
        return {"values": codecs.round_bf16(c), "codes": None, "scale": None}
    if store == "e4m3":
        amax = np.abs(c).max(axis=1)
        scale = codecs.round_f32(np.where(amax > 0, amax / codecs.E4M3_MAX, 1.0))
        r = codecs.round_e4m3(c / scale[:, None])
        return {"values": r * scale[:, None], "codes": codecs.e4m3_encode(r), "scale": scale}
    raise ValueError(store)


def store_keys(c, store: str) -> Dict[str, Optional[np.ndarray]]:
    """Indexer keys: like entries, but e4m3 keys carry no scale (saturating RNE of c),
    and "mxfp4" stores FP4 blocks of 32 channels with one power-of-two scale each
    (the indexer's FP4 keys: knightli.com DeepSeek-V4 KV-cache article, section
    "FP8 y FP4 reducen aun mas el costo de cache"; block format as in codecs).
    mxfp4 returns scale = the uint8 scale bytes [n][D/32]."""
    if store == "e4m3":
        r = codecs.round_e4m3(c)
        return {"values": r, "codes": codecs.e4m3_encode(r), "scale": None}
    if store == "mxfp4":
        values, codes, scale = codecs.mxfp4_quantize(c)
        return {"values": values, "codes": codes, "scale": scale}
    return store_entries(c, store)


# ---------------------------------------------------------------- lightning indexer + top-k
def index_scores(qI, w, keys) -> np.ndarray:
    """s_j = sum_h w_h * max(0, qI_h . key_j) for every row of `keys`.

    qI : [H_I][D_I], w : [H_I], keys : [n][D_I] (stored key values).  A score of
    exactly zero is returned as +0.0 (ReLU can zero every head term).
    """
    dots = np.asarray(keys, np.float64) @ np.asarray(qI, np.float64).T      # [n][H_I]
    s = np.maximum(dots, 0.0) @ np.asarray(w, np.float64)
    s[s == 0.0] = 0.0
    return s


def topk(scores, k: int) -> np.ndarray:
    """The min(k, n) best entries by (score descending, index ascending), returned as
    a set: ascending entry indices, padded with -1 to length k (int64)."""
    s = np.asarray(scores, np.float64)
    n = s.shape[0]
    kk = min(k, n)
    order = np.lexsort((np.arange(n), -s))       # primary: -s ascending; secondary: index
    out = np.full(k, -1, np.int64)
    out[:kk] = np.sort(order[:kk])
    return out


# ---------------------------------------------------------------- attention
def attend(q, items, tau: float):
    """Softmax attention of H query heads over n shared-latent items (K = V).

    q : [H][D], items : [n][D].  Returns (o [H][D], lse [H], p [H][n]).
    """
    q = np.asarray(q, np.float64)
    items = np.asarray(items, np.float64)
    logits = tau * (q @ items.T)
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    l = p.sum(axis=1, keepdims=True)
    p /= l
    return p @ items, (mx + np.log(l))[:, 0], p


def csa_row(t: int, q, qI, w, entries, keys, stream_v, m: int, W: int, k: int, tau: float):
    """One CSA query at position t of one sequence.

    entries, keys : stored (dequantised) caches [E][D], [E][D_I];
    stream_v : raw per-token latents [>= t+1][D] (the window source).
    Returns dict(e_vis, scores, idx, o, lse, p).
    """
    e_vis = min(entries_visible(t, m, W), entries.shape[0])
    s = index_scores(qI, w, keys[:e_vis])
    idx = topk(s, k)
    sel = idx[idx >= 0]
    items = np.concatenate([np.asarray(entries, np.float64)[sel],
                            np.asarray(np.asarray(stream_v)[window_positions(t, W)], np.float64)])
    o, lse, p = attend(q, items, tau)
    return {"e_vis": e_vis, "scores": s, "idx": idx, "o": o, "lse": lse, "p": p}


def hca_row(t: int, q, entries, stream_v, m: int, W: int, tau: float):
    """One HCA query at position t: dense over every visible entry plus the window."""
    e_vis = min(entries_visible(t, m, W), entries.shape[0])
    items = np.concatenate([np.asarray(entries, np.float64)[:e_vis],
                            np.asarray(np.asarray(stream_v)[window_positions(t, W)], np.float64)])
    o, lse, p = attend(q, items, tau)
    return {"e_vis": e_vis, "o": o, "lse": lse, "p": p}


# ---------------------------------------------------------------- projections of the hidden state
def project(x, W) -> np.ndarray:
    """A linear map of the rows of x: y = x W^T (x : [R][K], W : [N][K])."""
    return np.asarray(x, np.float64) @ np.asarray(W, np.float64).T


def absorb_queries(q_heads, W_UK) -> np.ndarray:
    """Queries against the shared latent: q~_h = (W_UK^h)^T q_h for every row and
    head (q_heads : [R][H][d_h], W_UK : [H][d_h][D] -> [R][H][D]); then
    q~_h . c = q_h . (W_UK^h c) for every latent c (MLA absorption)."""
    q_heads = np.asarray(q_heads, np.float64)
    W_UK = np.asarray(W_UK, np.float64)
    out = np.zeros((q_heads.shape[0], W_UK.shape[0], W_UK.shape[2]))
    for h in range(W_UK.shape[0]):
        out[:, h, :] = q_heads[:, h, :] @ W_UK[h]
    return out


# ---------------------------------------------------------------- heads back to the model width
def layer_output(o_latent, W_o, W_UV=None) -> np.ndarray:
    """y = W_o . concat_h(o_h) with o_h = W_UV^h o~_h when the latent is wider than
    the head dim (W_UV : [H][d_h][D]), else o_h = o~_h."""
    o_latent = np.asarray(o_latent, np.float64)
    if W_UV is not None:
        heads = np.einsum("hkd,hd->hk", np.asarray(W_UV, np.float64), o_latent)
    else:
        heads = o_latent
    return np.asarray(W_o, np.float64) @ heads.reshape(-1)


def attend_unabsorbed(q_heads, W_UK, W_UV, items, tau: float) -> np.ndarray:
    """Per-head keys k_h = W_UK^h c and values v_h = W_UV^h c formed explicitly
    (the form that latent absorption rewrites).  Returns o [H][d_h]."""
    items = np.asarray(items, np.float64)
    q_heads = np.asarray(q_heads, np.float64)
    H = q_heads.shape[0]
    out = np.empty((H, np.asarray(W_UV).shape[1]))
    for h in range(H):
        kh = items @ np.asarray(W_UK[h], np.float64).T        # [n][d_h]
        vh = items @ np.asarray(W_UV[h], np.float64).T
        lg = tau * (kh @ q_heads[h])
        p = np.exp(lg - lg.max())
        out[h] = (p / p.sum()) @ vh
    return out
