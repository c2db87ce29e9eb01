"""The five synthetic workloads of the CSA/HCA compressed-attention hot path.

Each workload is named by what it is and its sizes.  The layer kinds follow the
pages: CSA pools 4 tokens per entry over an overlapping window of 8 and keeps a
per-query top-k chosen by a lightning indexer; HCA pools 128 tokens per entry
and attends densely (knightli.com "DeepSeek-V4 KV cache" page, sections
"CSA: compresion 4x mas recuperacion dispersa" and "HCA: compresion 128x mas
atencion densa"); both add a raw window of the most recent 128 tokens (same
page, "Ventana deslizante").

Storage precisions: fp32 everywhere for the small CSA decode case; bf16 for
the others; the 1M-token pair stores entries in e4m3 with a per-entry fp32
scale and indexer keys in e4m3 (same page, "FP8 y FP4 reducen aun mas el costo
de cache").
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class LayerSpec:
    kind: str            # "csa" or "hca"
    m: int               # compression stride (tokens per entry)
    o: int               # extra leading tokens per pooling window (window = m + o)
    D: int               # shared latent dim of entries (K = V)
    H: int               # query heads
    d_h: int             # head dim before latent absorption
    W: int = 128         # raw sliding window
    H_I: int = 0         # indexer heads (CSA)
    D_I: int = 0         # indexer key/query dim (CSA)
    k: int = 0           # top-k (CSA)

    @property
    def absorbed(self) -> bool:
        """True when queries live in a latent wider than the head dim."""
        return self.D != self.d_h


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int                  # sequences
    N: int                  # tokens per sequence (decode: the query sits at t = N - 1)
    d_model: int
    layers: Tuple[LayerSpec, ...]
    mode: str               # "decode" (one query per sequence) or "prefill" (every token queries)
    store: str              # storage of per-token streams, queries and the window: "f32" | "bf16"
    entry_store: str        # "f32" | "bf16" | "e4m3" (e4m3 carries a per-entry fp32 scale)
    key_store: str          # "f32" | "bf16" | "e4m3" (unscaled)
    out_dtype: str          # "f32" | "bf16"
    heavy_frac: float = 0.0  # fraction of tokens whose hidden state is scaled by heavy_scale
    heavy_scale: float = 8.0
    description: str = ""

    def with_sizes(self, **kw) -> "Workload":
        """Same structure at other sizes (used for small parity cases)."""
        layers = kw.pop("layers", self.layers)
        lk = kw.pop("layer_kw", None)
        if lk:
            layers = tuple(replace(L, **lk) for L in layers)
        return replace(self, layers=layers, **kw)


CSA_DEC_4K_F32 = Workload(
    name="csa_decode_4k_f32", seed=0, B=1, N=4096, d_model=512,
    layers=(LayerSpec("csa", m=4, o=4, D=64, H=8, d_h=64, W=128, H_I=4, D_I=32, k=64),),
    mode="decode", store="f32", entry_store="f32", key_store="f32", out_dtype="f32",
    description="CSA decode, fp32, one query at t=4095 over a 4096-token prefix, batch 1")

HCA_DEC_64K_BF16 = Workload(
    name="hca_decode_64k_bf16", seed=1, B=4, N=65536, d_model=2048,
    layers=(LayerSpec("hca", m=128, o=0, D=128, H=32, d_h=128, W=128),),
    mode="decode", store="bf16", entry_store="bf16", key_store="bf16", out_dtype="f32",
    description="HCA decode, bf16 storage, fp32 accumulation, batch 4 at context 65536")

CSA_PREFILL_32K_BF16 = Workload(
    name="csa_prefill_32k_bf16", seed=2, B=1, N=32768, d_model=4096,
    layers=(LayerSpec("csa", m=4, o=4, D=512, H=64, d_h=128, W=128, H_I=64, D_I=128, k=512),),
    mode="prefill", store="bf16", entry_store="bf16", key_store="bf16", out_dtype="f32",
    heavy_frac=0.01, heavy_scale=8.0,
    description="CSA causal prefill, bf16, 32768 tokens, every token queries with top-512")

PAIR_DEC_128K_BF16 = Workload(
    name="pair_decode_128k_bf16", seed=3, B=32, N=131072, d_model=4096,
    layers=(LayerSpec("csa", m=4, o=4, D=512, H=64, d_h=128, W=128, H_I=64, D_I=128, k=1024),
            LayerSpec("hca", m=128, o=0, D=512, H=64, d_h=128, W=128)),
    mode="decode", store="bf16", entry_store="bf16", key_store="bf16", out_dtype="f32",
    description="interleaved CSA+HCA pair decode, batch 32 at context 131072, bf16 caches")

PAIR_DEC_1M_FP8 = Workload(
    name="pair_decode_1m_fp8", seed=4, B=1, N=1048576, d_model=4096,
    layers=(LayerSpec("csa", m=4, o=4, D=512, H=64, d_h=128, W=128, H_I=64, D_I=128, k=2048),
            LayerSpec("hca", m=128, o=0, D=512, H=64, d_h=128, W=128)),
    mode="decode", store="bf16", entry_store="e4m3", key_store="e4m3", out_dtype="bf16",
    description="interleaved CSA+HCA pair decode at context 1048576, e4m3 caches, bf16 query/output")

ALL = (CSA_DEC_4K_F32, HCA_DEC_64K_BF16, CSA_PREFILL_32K_BF16, PAIR_DEC_128K_BF16, PAIR_DEC_1M_FP8)
BY_NAME = {w.name: w for w in ALL}
