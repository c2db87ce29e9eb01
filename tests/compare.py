"""Comparison rules shared by the parity tests.

* top-k sets: equal, or every swapped pair is within the oracle's 1e-6 relative
  score gap; padding, order and visibility must match exactly.
* floating outputs: normwise max|g - o| <= rtol * max|o| (fp32 paths) or
  max|g - o| <= atol (bf16 / fp8 paths), against the unrounded fp64 oracle.
* stored codes (bf16 / e4m3 entries): equal, except one-step flips where the
  oracle's unrounded value lies within `mid_rtol` of a rounding midpoint.
"""
from __future__ import annotations

import numpy as np

SWAP_RTOL = 1e-6


def topk_parity(gpu_idx, ora_idx, ora_scores, rtol: float = SWAP_RTOL):
    """Returns (ok, message).  ora_scores: fp64 scores over the visible entries."""
    g = np.asarray(gpu_idx, np.int64)
    o = np.asarray(ora_idx, np.int64)
    if g.shape != o.shape:
        return False, f"shape {g.shape} vs {o.shape}"
    gv, ov = g[g >= 0], o[o >= 0]
    if len(gv) != len(ov):
        return False, f"{len(gv)} selected vs {len(ov)}"
    if not np.all(g[len(gv):] == -1):
        return False, "padding is not a -1 tail"
    if np.any(np.diff(gv) <= 0):
        return False, "indices not strictly ascending"
    n = len(ora_scores)
    if len(gv) and (gv.min() < 0 or gv.max() >= n):
        return False, "index outside the visible entries"
    if np.array_equal(gv, ov):
        return True, "exact"
    extra = np.setdiff1d(gv, ov)
    missing = np.setdiff1d(ov, gv)
    s = np.asarray(ora_scores, np.float64)
    for a in extra:
        for b in missing:
            if abs(s[a] - s[b]) > rtol * max(abs(s[a]), abs(s[b])):
                return False, f"illegal swap {a} ({s[a]!r}) for {b} ({s[b]!r})"
    return True, f"{len(extra)} allowed near-tie swaps"


def normwise(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    scale = float(np.max(np.abs(o))) if o.size else 0.0
    err = float(np.max(np.abs(g - o))) if o.size else 0.0
    return err, scale


def assert_close(g, o, *, rtol=None, atol=None, what=""):
    err, scale = normwise(g, o)
    if rtol is not None:
        assert err <= rtol * max(scale, 1e-30), f"{what}: max err {err:.3e} > {rtol} * {scale:.3e}"
    if atol is not None:
        assert err <= atol, f"{what}: max abs err {err:.3e} > {atol}"
    return err


def index_term_magnitude(q, w, keys):
    """Largest sum_h |w_h| max(0, q_h . k_j) over the keys: the size of the terms an
    indexer score adds up.  fp32 accumulation error scales with it, not with the
    score, which cancellation between heads of opposite weight can make small."""
    d = np.maximum(np.asarray(q, np.float64) @ np.asarray(keys, np.float64).T, 0.0)   # [H_I, E]
    return float(np.max(np.abs(np.asarray(w, np.float64)) @ d)) if d.size else 0.0


def assert_scores_close(g, o, q, w, keys, *, rtol, what=""):
    """Normwise check of indexer scores against the larger of max |score| and the
    term magnitude (index_term_magnitude)."""
    err, scale = normwise(g, o)
    scale = max(scale, index_term_magnitude(q, w, keys))
    assert err <= rtol * max(scale, 1e-30), f"{what}: max err {err:.3e} > {rtol} * {scale:.3e}"
    return err


def _spacing(y, sig_bits, min_normal_exp):
    """Distance between consecutive representable values around y (the larger one at a binade edge)."""
    _, e = np.frexp(np.asarray(y, np.float64))
    e = np.maximum(e, min_normal_exp + 1)
    return np.ldexp(1.0, e - sig_bits)


def rounding_mismatches(gpu_vals, ora_raw, ora_rounded, magnitude, fmt="bf16", rtol=1e-5):
    """Stored values that differ from the oracle's rounding, and how many of those
    are NOT a correct rounding of some value within rtol * magnitude of the oracle's
    unrounded value (`magnitude` = scale of the computation's rounding error; for
    a weighted sum sum_i p_i v_i it is sum_i p_i |v_i|).  Returns (n_diff, n_unexplained).
    """
    sig, emin = {"bf16": (8, -126), "e4m3": (4, -6)}[fmt]
    g = np.asarray(gpu_vals, np.float64)
    o = np.asarray(ora_rounded, np.float64)
    bad = g != o
    if not bad.any():
        return 0, 0
    gb = g[bad]
    raw = np.asarray(ora_raw, np.float64)[bad]
    mag = np.asarray(magnitude, np.float64)[bad]
    ok = np.abs(gb - raw) <= _spacing(gb, sig, emin) / 2 * (1 + 1e-12) + rtol * mag
    return int(bad.sum()), int((~ok).sum())


def bf16_code_flips(gpu_vals, ora_raw, ora_rounded, mid_rtol=1e-5, magnitude=None):
    """bf16 form of rounding_mismatches (magnitude defaults to |value|)."""
    mag = np.abs(np.asarray(ora_raw, np.float64)) if magnitude is None else magnitude
    return rounding_mismatches(gpu_vals, ora_raw, ora_rounded, mag, "bf16", mid_rtol)


def e4m3_flips(gpu_codes, ora_codes, ora_unrounded, magnitude, mid_rtol=1e-5):
    """e4m3 codes that differ from the oracle's, and those not explained by the GPU's
    fp32 error (within mid_rtol of `magnitude`) moving the value across a rounding boundary."""
    from oracle import codecs
    return rounding_mismatches(codecs.e4m3_decode(gpu_codes), ora_unrounded, codecs.e4m3_decode(ora_codes),
                               magnitude, "e4m3", mid_rtol)


def blocked_compress(v, g, bpos, m, o, block=16384):
    """oracle.method.compress over entry blocks: entry j reads only tokens
    [m j - o, m j + m), so each block runs on its own token slice (bounded host
    memory at million-token sizes).  Needs o % m == 0."""
    import numpy as np

    from oracle import method
    assert o % m == 0
    N = v.shape[0]
    E = N // m
    out = []
    for j0 in range(0, E, block):
        j1 = min(E, j0 + block)
        t0 = max(0, m * j0 - o)
        c = method.compress(v[t0:m * j1], g[t0:m * j1], bpos, m, o)
        out.append(c if j0 == 0 else c[o // m:])
    return np.concatenate(out) if out else np.zeros((0, v.shape[1]))


def mxfp4_flips(gpu_codes, gpu_scale, ora_unrounded, magnitude, rtol=1e-5):
    """MXFP4 blocks stored by the GPU against the oracle's rounding of the unrounded
    values c [n][D] (magnitude [n][D]: scale of the GPU's fp32 error in c).  A block
    scale is explained when it is the oracle's scale rule applied to some block
    maximum within rtol * (block's largest magnitude) of the oracle's; an element
    is explained when, under the GPU's scale, it lies between the roundings of
    c - rtol * mag and c + rtol * mag (rounding is monotone).  Returns
    (elements or scales that differ from the oracle's, how many are unexplained)."""
    from oracle import codecs
    c = np.asarray(ora_unrounded, np.float64)
    mag = np.asarray(magnitude, np.float64)
    n, D = c.shape
    _, o_codes, o_scale = codecs.mxfp4_quantize(c)
    gc = np.asarray(gpu_codes).astype(np.int64)
    gs = np.asarray(gpu_scale).astype(np.int64)
    nb = D // codecs.MX_BLOCK
    cb = c.reshape(n, nb, codecs.MX_BLOCK)
    d = rtol * mag.reshape(n, nb, codecs.MX_BLOCK)

    def rule(amax):
        _, e = np.frexp(np.where(amax > 0, amax, 1.0))
        return np.clip(np.where(amax > 0, e - 3, -127), -127, 127) + 127

    amax = np.abs(cb).max(axis=2)
    slack = d.max(axis=2)
    lo_s, hi_s = rule(np.maximum(amax - slack, 0.0)), rule(amax + slack)
    scale_diff = gs != o_scale
    scale_bad = (gs < lo_s) | (gs > hi_s)
    X = np.ldexp(1.0, gs - 127)[:, :, None]
    g_val = codecs.e2m1_decode(gc).reshape(n, nb, codecs.MX_BLOCK)
    lo = codecs.round_e2m1((cb - d) / X)
    hi = codecs.round_e2m1((cb + d) / X)
    elem_diff = (gc != o_codes.astype(np.int64)).reshape(n, nb, codecs.MX_BLOCK) & \
        ~((g_val == 0) & (codecs.e2m1_decode(o_codes).reshape(n, nb, codecs.MX_BLOCK) == 0) & ~scale_diff[:, :, None])
    elem_bad = elem_diff & ((g_val < lo) | (g_val > hi))
    return int(scale_diff.sum() + elem_diff.sum()), int(scale_bad.sum() + elem_bad.sum())
