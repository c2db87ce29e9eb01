"""Seeded synthetic inputs for the CSA/HCA hot path.

This module only draws random numbers and forms the caller-side inputs of the
library from them: hidden states x ~ N(0, 1), weights ~ N(0, 1/fan_in), the
per-token projections (value and gate streams, queries) and their rounding to
the storage precision.  None of the method's own steps (pooling, indexing,
selection, attention) lives here; the oracle and the HIP path both start from
these arrays.

Reproducibility: every array comes from its own numpy SeedSequence, keyed by
(workload seed, purpose, indices), so any slice can be regenerated alone:
  weights       spawn_key (0, layer, weight number)
  hidden state  spawn_key (1, sequence, 4096-token chunk)
  heavy tokens  spawn_key (2, sequence)
Chunks are drawn on a thread pool; the values do not depend on the pool size.

Values in storage precision are returned as float32 arrays holding exactly
representable values (bf16 values are exact in float32), so the host side
never needs a bf16 numpy type.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

from .configs import LayerSpec, Workload

CHUNK_TOKENS = 4096

_WEIGHT_IDS = {"W_c": 0, "W_g": 1, "bpos": 2, "W_cI": 3, "W_gI": 4, "bposI": 5,
               "W_q": 6, "W_UK": 7, "W_UV": 8, "W_iq": 9, "W_w": 10, "W_o": 11}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key)))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def round_store(x: np.ndarray, store: str) -> np.ndarray:
    """Round to the storage precision with round-to-nearest-even (torch's CPU cast)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if store == "f32":
        return x
    if store == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(store)


def torch_dtype(store: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[store]


# ---------------------------------------------------------------- weights
def weight(wl: Workload, li: int, name: str) -> np.ndarray:
    """One weight of layer `li`, float32, ~ N(0, 1/fan_in)."""
    L = wl.layers[li]
    dm = wl.d_model
    shapes = {
        "W_c": ((L.D, dm), dm), "W_g": ((L.D, dm), dm),
        # the position bias has no fan-in of its own: it uses that of the gate it biases
        "bpos": ((L.m + L.o, L.D), dm),
        "W_cI": ((L.D_I, dm), dm), "W_gI": ((L.D_I, dm), dm), "bposI": ((L.m + L.o, L.D_I), dm),
        "W_q": ((L.H * L.d_h, dm), dm),
        "W_UK": ((L.H, L.d_h, L.D), L.D), "W_UV": ((L.H, L.d_h, L.D), L.D),
        "W_iq": ((L.H_I * L.D_I, dm), dm), "W_w": ((L.H_I, dm), dm),
        "W_o": ((dm, L.H * L.d_h), L.H * L.d_h),
    }
    shape, fan_in = shapes[name]
    r = _rng(wl.seed, 0, li, _WEIGHT_IDS[name])
    w = r.standard_normal(shape, dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(fan_in))
    return w


def layer_weights(wl: Workload, li: int) -> Dict[str, np.ndarray]:
    L = wl.layers[li]
    names = ["W_c", "W_g", "bpos", "W_q", "W_o"]
    if L.absorbed:
        names += ["W_UK", "W_UV"]
    if L.kind == "csa":
        names += ["W_cI", "W_gI", "bposI", "W_iq", "W_w"]
    return {n: weight(wl, li, n) for n in names}


# ---------------------------------------------------------------- hidden states
def heavy_positions(wl: Workload, b: int) -> np.ndarray:
    """Token positions of sequence b whose whole hidden vector is scaled."""
    n = int(round(wl.heavy_frac * wl.N))
    if n == 0:
        return np.zeros(0, np.int64)
    return np.sort(_rng(wl.seed, 2, b).choice(wl.N, size=n, replace=False))


def hidden_states(wl: Workload, b: int, t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
    """x[t0:t1] of sequence b, float32 [t1 - t0][d_model]."""
    t1 = wl.N if t1 is None else t1
    assert 0 <= t0 <= t1 <= wl.N
    c0, c1 = t0 // CHUNK_TOKENS, (t1 + CHUNK_TOKENS - 1) // CHUNK_TOKENS
    out = np.empty((t1 - t0, wl.d_model), np.float32)

    def fill(c):
        a, e = c * CHUNK_TOKENS, min(wl.N, (c + 1) * CHUNK_TOKENS)
        blk = _rng(wl.seed, 1, b, c).standard_normal((e - a, wl.d_model), dtype=np.float32)
        lo, hi = max(a, t0), min(e, t1)
        out[lo - t0:hi - t0] = blk[lo - a:hi - a]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(c0, c1)))
    hp = heavy_positions(wl, b)
    hp = hp[(hp >= t0) & (hp < t1)]
    if hp.size:
        out[hp - t0] *= np.float32(wl.heavy_scale)
    return out


def _project(x: np.ndarray, W: np.ndarray, rows_per_task: int = 8192) -> np.ndarray:
    """x @ W.T in float32 (BLAS), in row blocks to bound temporaries."""
    out = np.empty((x.shape[0], W.shape[0]), np.float32)
    for a in range(0, x.shape[0], rows_per_task):
        np.matmul(x[a:a + rows_per_task], W.T, out=out[a:a + rows_per_task])
    return out


# ---------------------------------------------------------------- streams and queries
def layer_streams(wl: Workload, li: int, x: np.ndarray, weights=None) -> Dict[str, np.ndarray]:
    """Per-token value/gate streams of layer li for hidden states x [n][d_model],
    rounded to storage: v, g [n][D] and (CSA) vI, gI [n][D_I]."""
    L = wl.layers[li]
    w = weights if weights is not None else layer_weights(wl, li)
    out = {"v": round_store(_project(x, w["W_c"]), wl.store),
           "g": round_store(_project(x, w["W_g"]), wl.store)}
    if L.kind == "csa":
        out["vI"] = round_store(_project(x, w["W_cI"]), wl.store)
        out["gI"] = round_store(_project(x, w["W_gI"]), wl.store)
    return out


def layer_queries(wl: Workload, li: int, x_rows: np.ndarray, weights=None) -> Dict[str, np.ndarray]:
    """Queries of layer li for the hidden states of the query rows x_rows [R][d_model].

    q_heads [R][H][d_h] float32: per-head queries before absorption (unrounded);
    q       [R][H][D]   stored:  the query against the shared latent; equal to q_heads
                                 when D == d_h, else W_UK^h^T q_h (latent absorption);
    qI      [R][H_I][D_I] stored, w [R][H_I] float32 (CSA only).
    """
    L = wl.layers[li]
    w = weights if weights is not None else layer_weights(wl, li)
    R = x_rows.shape[0]
    qh = _project(x_rows, w["W_q"]).reshape(R, L.H, L.d_h)
    if L.absorbed:
        # [R][H][d_h] x [H][d_h][D] -> [R][H][D], one batched product per head
        qt = np.einsum("rhk,hkd->rhd", qh, w["W_UK"], optimize=True).astype(np.float32)
    else:
        qt = qh
    out = {"q_heads": qh, "q": round_store(qt, wl.store)}
    if L.kind == "csa":
        out["qI"] = round_store(_project(x_rows, w["W_iq"]).reshape(R, L.H_I, L.D_I), wl.store)
        out["w"] = _project(x_rows, w["W_w"]).astype(np.float32)
    return out


def decode_inputs(wl: Workload, b: int, x: Optional[np.ndarray] = None) -> Dict:
    """Everything one decode sequence b needs on the host: its hidden states,
    per-layer streams, and per-layer queries of the single row at t = N - 1."""
    assert wl.mode == "decode"
    x = hidden_states(wl, b) if x is None else x
    layers = []
    for li in range(len(wl.layers)):
        w = layer_weights(wl, li)
        st = layer_streams(wl, li, x, w)
        q = layer_queries(wl, li, x[wl.N - 1:wl.N], w)
        layers.append({"weights": w, "streams": st, "queries": q})
    return {"t": wl.N - 1, "layers": layers}


# ---------------------------------------------------------------- GPU-side synthesis (same recipe, torch RNG)
def gpu_weights(wl: Workload, device, seed_offset: int = 0):
    """Per-layer projection weights drawn on the GPU with torch's RNG (fp32)."""
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000003 + 7919 + seed_offset)
    dm = wl.d_model
    out = []
    for L in wl.layers:
        names = [("v", L.D), ("g", L.D)] + ([("vI", L.D_I), ("gI", L.D_I)] if L.kind == "csa" else [])
        w = {n: torch.randn(r, dm, device=device, generator=g) * (1.0 / math.sqrt(dm)) for n, r in names}
        w["bpos"] = torch.randn(L.m + L.o, L.D, device=device, generator=g) * (1.0 / math.sqrt(dm))
        if L.kind == "csa":
            w["bposI"] = torch.randn(L.m + L.o, L.D_I, device=device, generator=g) * (1.0 / math.sqrt(dm))
        out.append(w)
    return out


def _gpu_hidden_chunk(wl: Workload, b: int, g, a: int, e: int, device):
    """x[a:e] of sequence b drawn with the GPU generator g (consumed in order),
    with the heavy-token scaling of the host recipe at the same positions."""
    x = torch.randn(e - a, wl.d_model, device=device, generator=g)
    hp = heavy_positions(wl, b)
    hp = hp[(hp >= a) & (hp < e)]
    if hp.size:
        x[torch.from_numpy(hp - a).to(device)] *= wl.heavy_scale
    return x


def gpu_sequence_streams(wl: Workload, b: int, weights, device, chunk: int = 32768):
    """Streams of every layer for sequence b, from one hidden-state stream drawn on
    the GPU with torch's RNG (x ~ N(0,1), heavy tokens scaled as in the host
    recipe; fp32 projections rounded to storage).

    Same distributions as the host recipe, other random numbers: the inputs of
    the full-size runs (timed decode steps, and the full-size parity tests, which
    copy the streams of sampled sequences back to the host for the oracle).
    Returns a list (per layer) of dicts of torch tensors [N][D] in storage dtype.
    """
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000003 + 104729 * (b + 1))
    dt = torch_dtype(wl.store)
    out = []
    for L, w in zip(wl.layers, weights):
        names = ["v", "g"] + (["vI", "gI"] if L.kind == "csa" else [])
        out.append({n: torch.empty(wl.N, w[n].shape[0], device=device, dtype=dt) for n in names})
    for a in range(0, wl.N, chunk):
        e = min(wl.N, a + chunk)
        x = _gpu_hidden_chunk(wl, b, g, a, e, device)
        for st, w in zip(out, weights):
            for n in st:
                st[n][a:e] = (x @ w[n].T).to(dt)
    return out


def gpu_prefill_inputs(wl: Workload, device, chunk: int = 4096):
    """Prefill inputs of layer 0 for sequence 0 drawn on the GPU: the streams and,
    from the same hidden state x_t, the query of every row t (causal prefill).

    Returns (weights, streams, queries): streams as gpu_sequence_streams (layer 0),
    queries {q [N][H][D] (absorbed when D != d_h), qI [N][H_I][D_I]} in storage
    dtype and w [N][H_I] fp32.
    """
    L = wl.layers[0]
    weights = gpu_weights(wl, device)
    w0 = weights[0]
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000003 + 15485863)
    dm = wl.d_model
    dt = torch_dtype(wl.store)
    Wq = torch.randn(L.H * L.d_h, dm, device=device, generator=g) / math.sqrt(dm)
    WUK = (torch.randn(L.H, L.d_h, L.D, device=device, generator=g) / math.sqrt(L.D)) if L.absorbed else None
    Wiq = torch.randn(L.H_I * L.D_I, dm, device=device, generator=g) / math.sqrt(dm)
    Ww = torch.randn(L.H_I, dm, device=device, generator=g) / math.sqrt(dm)
    names = ["v", "g", "vI", "gI"]
    st = {n: torch.empty(wl.N, w0[n].shape[0], device=device, dtype=dt) for n in names}
    q = torch.empty(wl.N, L.H, L.D, device=device, dtype=dt)
    qI = torch.empty(wl.N, L.H_I, L.D_I, device=device, dtype=dt)
    w = torch.empty(wl.N, L.H_I, device=device, dtype=torch.float32)
    gx = torch.Generator(device=device)
    gx.manual_seed(wl.seed * 1000003 + 104729)
    for a in range(0, wl.N, chunk):
        e = min(wl.N, a + chunk)
        x = _gpu_hidden_chunk(wl, 0, gx, a, e, device)
        for n in names:
            st[n][a:e] = (x @ w0[n].T).to(dt)
        qh = (x @ Wq.T).view(e - a, L.H, L.d_h)
        if WUK is not None:
            qt = torch.bmm(qh.transpose(0, 1).contiguous(), WUK).transpose(0, 1)
        else:
            qt = qh
        q[a:e] = qt.to(dt)
        qI[a:e] = (x @ Wiq.T).view(e - a, L.H_I, L.D_I).to(dt)
        w[a:e] = x @ Ww.T
    return weights, st, {"q": q, "qI": qI, "w": w}


def gpu_queries(wl: Workload, li: int, R: int, device, seed_offset: int = 0):
    """Random queries for R rows on the GPU (same distributions as layer_queries)."""
    L = wl.layers[li]
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000003 + li * 7919 + 104729 + seed_offset)
    dm = wl.d_model
    dt = torch_dtype(wl.store)
    x = torch.randn(R, dm, device=device, generator=g)
    Wq = torch.randn(L.H * L.d_h, dm, device=device, generator=g) / math.sqrt(dm)
    qh = (x @ Wq.T).view(R, L.H, L.d_h)
    if L.absorbed:
        WUK = torch.randn(L.H, L.d_h, L.D, device=device, generator=g) / math.sqrt(L.D)
        qt = torch.bmm(qh.transpose(0, 1).contiguous(), WUK).transpose(0, 1).contiguous()
    else:
        qt = qh
    out = {"q": qt.to(dt).contiguous()}
    if L.kind == "csa":
        Wiq = torch.randn(L.H_I * L.D_I, dm, device=device, generator=g) / math.sqrt(dm)
        Ww = torch.randn(L.H_I, dm, device=device, generator=g) / math.sqrt(dm)
        out["qI"] = (x @ Wiq.T).view(R, L.H_I, L.D_I).to(dt).contiguous()
        out["w"] = (x @ Ww.T).float().contiguous()
    return out
