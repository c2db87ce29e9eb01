"""Helpers of the GPU parity tests: uploads and small synthetic caches."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def dev(a, store: str = "f32") -> torch.Tensor:
    """Upload float32 values (already exact in `store`) in that storage dtype."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    if store == "bf16":
        t = t.to(torch.bfloat16)
    return t.contiguous()


def dev_codes(codes) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(DEV).view(torch.float8_e4m3fn)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.int32 else t.cpu().numpy()


def rng_store(rng, shape, store: str, scale: float = 1.0) -> np.ndarray:
    """Random N(0, scale^2) values exact in the storage dtype (float32 array)."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    if store == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    return x
