"""A workload layer end to end on the CPU: caches from streams, then decode rows.

TEST INFRASTRUCTURE ONLY (see the package header).  Sources as in method.py.
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np

from . import method


def tau(d_h: int) -> float:
    """Softmax scale 1/sqrt(d_h) of the un-absorbed heads (kept under absorption)."""
    return 1.0 / math.sqrt(d_h)


def layer_caches(L, streams: Dict[str, np.ndarray], weights: Dict[str, np.ndarray],
                 entry_store: str, key_store: str) -> Dict[str, Dict]:
    """Compress one sequence's streams into stored entries (and CSA indexer keys)."""
    c = method.compress(streams["v"], streams["g"], weights["bpos"], L.m, L.o)
    out = {"entries": method.store_entries(c, entry_store), "entries_raw": c}
    if L.kind == "csa":
        kI = method.compress(streams["vI"], streams["gI"], weights["bposI"], L.m, L.o)
        out["keys"] = method.store_keys(kI, key_store)
        out["keys_raw"] = kI
    return out


def decode_row(L, caches, stream_v, q, t: int, qI=None, w=None) -> Dict:
    """One query row of layer L at position t against stored caches."""
    ent = caches["entries"]["values"]
    if L.kind == "csa":
        return method.csa_row(t, q, qI, w, ent, caches["keys"]["values"], stream_v,
                              L.m, L.W, L.k, tau(L.d_h))
    return method.hca_row(t, q, ent, stream_v, L.m, L.W, tau(L.d_h))
