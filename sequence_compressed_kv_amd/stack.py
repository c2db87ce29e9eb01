"""A multi-layer stack of compressed-attention layers on the library's calls.

The hybrid schedule: two HCA layers, then CSA and HCA alternating (knightli.com
DeepSeek-V4 KV-cache article, section "Pila hibrida de capas").  Layer l's output
rows are layer l + 1's hidden rows; the norms, residual adds and MLPs of a model
are not part of the attention path and are left out.  This module is host-side
orchestration only: every product, pool, score, selection and softmax runs in the
library's kernels.

Memory plan: the caches of all layers (pooled entries, indexer key tiles, the
window ring that doubles as the value ring, the gate ring and the indexer's two
rings) are carved from one device arena, each buffer 256-byte aligned; `plan`
lists them with their offsets.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import torch

from . import _lib as sk


@dataclass(frozen=True)
class StackLayer:
    kind: str        # "csa" or "hca"
    m: int           # tokens per entry
    o: int           # extra leading tokens of a pooling window
    D: int           # shared latent
    H: int           # query heads
    d_h: int         # head dim (absorbed into the latent when D != d_h)
    W: int = 128     # raw window
    H_I: int = 0     # indexer heads (CSA)
    D_I: int = 0     # indexer dim (CSA)
    k: int = 0       # top-k (CSA)
    keys: str = "bf16"   # indexer key storage (CSA): "bf16" key tiles or "mxfp4" FP4 blocks


def hybrid_schedule(n_layers: int, csa: StackLayer, hca: StackLayer) -> List[StackLayer]:
    """HCA, HCA, then CSA / HCA alternating."""
    return [hca if i < 2 or (i - 2) % 2 == 1 else csa for i in range(n_layers)]


def layer_weight_shapes(L: StackLayer, d_model: int) -> Dict[str, tuple]:
    """Weights of one layer (all bf16 except the fp32 position biases)."""
    s = {"W_q": (L.H * L.d_h, d_model), "W_o": (d_model, L.H * L.d_h), "W_c": (L.D, d_model),
         "W_g": (L.D, d_model), "bpos": (L.m + L.o, L.D)}
    if L.D != L.d_h:
        s["W_UK"] = (L.H, L.d_h, L.D)
        s["W_UV"] = (L.H, L.d_h, L.D)
    if L.kind == "csa":
        s.update({"W_iq": (L.H_I * L.D_I, d_model), "W_w": (L.H_I, d_model), "W_cI": (L.D_I, d_model),
                  "W_gI": (L.D_I, d_model), "bposI": (L.m + L.o, L.D_I)})
    return s


class Arena:
    """One device allocation carved into 256-byte aligned buffers."""

    def __init__(self, device):
        self.device = device
        self.items = []      # (name, offset, nbytes, shape, dtype)
        self.size = 0
        self.buf: Optional[torch.Tensor] = None

    def reserve(self, name: str, shape, dtype) -> int:
        nbytes = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        off = (self.size + 255) // 256 * 256
        self.items.append((name, off, nbytes, tuple(shape), dtype))
        self.size = off + nbytes
        return len(self.items) - 1

    def allocate(self):
        self.buf = torch.empty(max(self.size, 1), dtype=torch.uint8, device=self.device)

    def view(self, i: int) -> torch.Tensor:
        _, off, nbytes, shape, dtype = self.items[i]
        return self.buf[off:off + nbytes].view(dtype).view(shape)


class Stack:
    """Caches of B sequences of up to N_max tokens for every layer, and the two ways
    through the stack: prefill (every token of the sequences, causal rows) and a
    decode step (one new token per sequence)."""

    def __init__(self, layers: Sequence[StackLayer], weights: Sequence[Dict[str, torch.Tensor]], d_model: int,
                 B: int, N_max: int, device="cuda:0"):
        self.layers, self.weights = list(layers), list(weights)
        self.d_model, self.B, self.N_max, self.device = d_model, B, N_max, device
        bf = torch.bfloat16
        arena = Arena(device)
        self._slots = []
        for li, L in enumerate(self.layers):
            if L.W < L.m + L.o:
                raise ValueError(f"layer {li}: the window ring (W={L.W}) must hold a pooling window ({L.m + L.o})")
            E_cap = N_max // L.m
            sl = {"entries": arena.reserve(f"{li}.entries", (B, E_cap, L.D), bf),
                  "win": arena.reserve(f"{li}.window_ring", (B, L.W, L.D), bf),
                  "g_ring": arena.reserve(f"{li}.gate_ring", (B, L.W, L.D), bf)}
            if L.kind == "csa":
                E_t = (E_cap + 31) // 32 * 32
                if L.keys == "mxfp4":
                    sl["keys"] = arena.reserve(f"{li}.index_keys", (B, E_t // 32, 17 * L.D_I), torch.uint8)
                elif L.keys == "bf16":
                    sl["keys"] = arena.reserve(f"{li}.index_keys", (B, E_t // 32, L.D_I // 8, 32, 8), bf)
                else:
                    raise ValueError(f"layer {li}: unknown key storage {L.keys!r}")
                sl["vI_ring"] = arena.reserve(f"{li}.index_value_ring", (B, L.m + L.o, L.D_I), bf)
                sl["gI_ring"] = arena.reserve(f"{li}.index_gate_ring", (B, L.m + L.o, L.D_I), bf)
            self._slots.append(sl)
        arena.allocate()
        self.arena = arena
        self.caches = [{k: arena.view(i) for k, i in sl.items()} for sl in self._slots]
        for L, c in zip(self.layers, self.caches):
            if L.kind == "csa" and L.keys == "mxfp4":
                c["keys"] = sk.Mxfp4Keys(c["keys"], L.D_I)
        self._decode_ws: Optional[List[Dict]] = None

    @property
    def plan(self):
        """(buffer, offset, bytes) of every cache buffer in the arena."""
        return [(n, off, nb) for n, off, nb, _, _ in self.arena.items]

    # ------------------------------------------------------------ pieces of one layer
    def _inputs(self, li, x, R, ws=None):
        """layer_inputs of layer li for rows x [R][d_model]: queries and streams."""
        L, w = self.layers[li], self.weights[li]
        bf = torch.bfloat16
        t = {"q": torch.empty(R, L.H, L.D, device=self.device, dtype=bf),
             "v": torch.empty(R, L.D, device=self.device, dtype=bf), "g": torch.empty(R, L.D, device=self.device, dtype=bf)}
        kw = dict(W_UK=w.get("W_UK"), W_c=w["W_c"], v=t["v"], W_g=w["W_g"], g=t["g"])
        if L.kind == "csa":
            t.update({"qI": torch.empty(R, L.H_I, L.D_I, device=self.device, dtype=bf),
                      "w": torch.empty(R, L.H_I, device=self.device),
                      "vI": torch.empty(R, L.D_I, device=self.device, dtype=bf),
                      "gI": torch.empty(R, L.D_I, device=self.device, dtype=bf)})
            kw.update(W_iq=w["W_iq"], qI=t["qI"], W_w=w["W_w"], w=t["w"], W_cI=w["W_cI"], vI=t["vI"], W_gI=w["W_gI"],
                      gI=t["gI"])
        t["ws"] = sk.layer_inputs(x, w["W_q"], t["q"], workspace=ws, **kw)
        return t

    def _tau(self, L):
        return 1.0 / math.sqrt(L.d_h)

    # ------------------------------------------------------------ prefill
    def prefill(self, x: torch.Tensor, out_dtype=torch.bfloat16, record: Optional[list] = None) -> List[torch.Tensor]:
        """x [B][N][d_model] bf16, N <= N_max: every token of every sequence through
        the stack (causal rows).  Fills every layer's caches and rings; returns each
        layer's output rows [B][N][d_model].  With a list as `record`, each layer
        appends its intermediates: the projections' outputs ("t": q, v, g and for CSA
        qI, w, vI, gI, rows b * N + position), the selections ("idx": per sequence
        [N][k], CSA) and the attention outputs ("o" [B * N][H][D])."""
        B, N, dm = x.shape
        assert B == self.B and N <= self.N_max and dm == self.d_model
        outs = []
        h = x.reshape(B * N, dm)
        for li, L in enumerate(self.layers):
            c, w = self.caches[li], self.weights[li]
            t = self._inputs(li, h, B * N)
            v, g = t["v"].view(B, N, L.D), t["g"].view(B, N, L.D)
            kv = sk.Pool(v, g, w["bpos"], c["entries"])
            if L.kind == "csa":
                vI, gI = t["vI"].view(B, N, L.D_I), t["gI"].view(B, N, L.D_I)
                sk.csa_compress(kv, sk.Pool(vI, gI, w["bposI"], c["keys"], layout=sk.LAYOUT_KEY_TILES), m=L.m, o=L.o)
            else:
                sk.hca_compress(kv, m=L.m, o=L.o)
            self._fill_rings(li, t, B, N)
            o = torch.empty(B * N, L.H, L.D, device=self.device, dtype=torch.bfloat16)
            kept = []
            for b in range(B):
                rows = sk.RowSpec.causal(N, seq0=b)
                r = slice(b * N, (b + 1) * N)
                if L.kind == "csa":
                    idx = torch.empty(N, L.k, dtype=torch.int32, device=self.device)
                    sk.csa_index_topk(rows, t["qI"][r], t["w"][r], c["keys"], idx, m=L.m, W=L.W, k=L.k)
                    sk.csa_attend(rows, t["q"][r], c["entries"], idx, v, o[r], m=L.m, W=L.W,
                                  softmax_scale=self._tau(L))
                    kept.append(idx)
                else:
                    sk.hca_attend(rows, t["q"][r], c["entries"], v, o[r], m=L.m, W=L.W, softmax_scale=self._tau(L))
            y = torch.empty(B * N, dm, device=self.device, dtype=out_dtype)
            sk.layer_output(o, w["W_o"], y, W_UV=w.get("W_UV"))
            outs.append(y.view(B, N, dm))
            if record is not None:
                record.append({"t": t, "idx": kept, "o": o})
            h = y if out_dtype == torch.bfloat16 else y.to(torch.bfloat16)
        return outs

    def _fill_rings(self, li, t, B, N):
        """The rings as a decode step at position N would find them: slot = position
        mod ring length, for the last ring-length tokens."""
        L, c = self.layers[li], self.caches[li]
        pos = torch.arange(max(0, N - L.W), N, device=self.device)
        c["win"][:, pos % L.W] = t["v"].view(B, N, L.D)[:, pos]
        c["g_ring"][:, pos % L.W] = t["g"].view(B, N, L.D)[:, pos]
        if L.kind == "csa":
            P = L.m + L.o
            pi = torch.arange(max(0, N - P), N, device=self.device)
            c["vI_ring"][:, pi % P] = t["vI"].view(B, N, L.D_I)[:, pi]
            c["gI_ring"][:, pi % P] = t["gI"].view(B, N, L.D_I)[:, pi]

    # ------------------------------------------------------------ decode
    def decode(self, x: torch.Tensor, pos: torch.Tensor, out_dtype=torch.bfloat16) -> List[torch.Tensor]:
        """One new token per sequence: x [B][d_model] bf16 at positions pos [B] (int32,
        each below N_max).  Appends every layer's token, then attends; returns each
        layer's output rows [B][d_model].  Workspaces and outputs are allocated on the
        first call and reused, so later calls allocate nothing (HIP-graph capturable)."""
        B = self.B
        first = self._decode_ws is None
        if first:
            self._decode_ws = [dict() for _ in self.layers]
        rows = sk.RowSpec.decode(pos, self.N_max - 1)
        h = x
        outs = []
        for li, L in enumerate(self.layers):
            c, w, st = self.caches[li], self.weights[li], self._decode_ws[li]
            if first:
                st["t"] = self._inputs(li, h, B)
                st["o"] = torch.empty(B, L.H, L.D, device=self.device, dtype=torch.bfloat16)
                st["y"] = torch.empty(B, self.d_model, device=self.device, dtype=out_dtype)
                if L.kind == "csa":
                    st["idx"] = torch.empty(B, L.k, dtype=torch.int32, device=self.device)
            else:
                self._inputs_into(li, h, st["t"])
            t = st["t"]
            kv = sk.Append(pos, t["v"], t["g"], c["win"], c["g_ring"], w["bpos"], c["entries"])
            if L.kind == "csa":
                sk.csa_append(kv, sk.Append(pos, t["vI"], t["gI"], c["vI_ring"], c["gI_ring"], w["bposI"], c["keys"],
                                            layout=sk.LAYOUT_KEY_TILES), m=L.m, o=L.o)
                st["ws_i"] = sk.csa_index_topk(rows, t["qI"], t["w"], c["keys"], st["idx"], m=L.m, W=L.W, k=L.k,
                                               workspace=st.get("ws_i"))
                st["ws_a"] = sk.csa_attend(rows, t["q"], c["entries"], st["idx"], c["win"], st["o"], m=L.m, W=L.W,
                                           softmax_scale=self._tau(L), workspace=st.get("ws_a"))
            else:
                sk.hca_append(kv, m=L.m, o=L.o)
                st["ws_a"] = sk.hca_attend(rows, t["q"], c["entries"], c["win"], st["o"], m=L.m, W=L.W,
                                           softmax_scale=self._tau(L), workspace=st.get("ws_a"))
            st["ws_o"] = sk.layer_output(st["o"], w["W_o"], st["y"], W_UV=w.get("W_UV"), workspace=st.get("ws_o"))
            outs.append(st["y"])
            h = st["y"] if out_dtype == torch.bfloat16 else st["y"].to(torch.bfloat16)
        return outs

    def _inputs_into(self, li, x, t):
        L, w = self.layers[li], self.weights[li]
        kw = dict(W_UK=w.get("W_UK"), W_c=w["W_c"], v=t["v"], W_g=w["W_g"], g=t["g"])
        if L.kind == "csa":
            kw.update(W_iq=w["W_iq"], qI=t["qI"], W_w=w["W_w"], w=t["w"], W_cI=w["W_cI"], vI=t["vI"], W_gI=w["W_gI"],
                      gI=t["gI"])
        sk.layer_inputs(x, w["W_q"], t["q"], workspace=t["ws"], **kw)
