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


def bf16_code_flips(gpu_vals, ora_raw, ora_rounded, mid_rtol=1e-5, magnitude=None):
    """Count bf16 code mismatches, and those not explained by a near-midpoint value.

    A mismatch is explained when the codes are one step apart and the oracle's
    unrounded value lies within mid_rtol * magnitude of the midpoint between them;
    `magnitude` is the scale of the rounding error of the value's computation
    (for a weighted sum sum_i p_i v_i it is sum_i p_i |v_i|), default |value|.
    """
    from oracle import codecs  # test infrastructure
    g = codecs.bf16_bits(gpu_vals).astype(np.int64)
    o = codecs.bf16_bits(ora_rounded).astype(np.int64)
    bad = g != o
    if not bad.any():
        return 0, 0
    raw = np.asarray(ora_raw, np.float64)[bad]
    mag = np.abs(raw) if magnitude is None else np.asarray(magnitude, np.float64)[bad]
    gv = np.asarray(gpu_vals, np.float64)[bad]
    ov = np.asarray(ora_rounded, np.float64)[bad]
    mid = (gv + ov) / 2
    near_mid = np.abs(raw - mid) <= mid_rtol * mag
    one_step = np.abs(g[bad] - o[bad]) == 1
    return int(bad.sum()), int((~(near_mid & one_step)).sum())
