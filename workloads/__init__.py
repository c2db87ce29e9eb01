"""Seeded synthetic workloads (shapes, distributions, caller-side projections).

Shared by the oracle-side tests and the HIP-side tests and bench; holds none of
the compressed-attention method's own arithmetic.
"""
from .configs import (ALL, BY_NAME, CSA_DEC_4K_F32, CSA_PREFILL_32K_BF16, HCA_DEC_64K_BF16,
                      PAIR_DEC_128K_BF16, PAIR_DEC_1M_FP8, LayerSpec, Workload)
from . import gen

__all__ = ["ALL", "BY_NAME", "CSA_DEC_4K_F32", "HCA_DEC_64K_BF16", "CSA_PREFILL_32K_BF16",
           "PAIR_DEC_128K_BF16", "PAIR_DEC_1M_FP8", "LayerSpec", "Workload", "gen"]
