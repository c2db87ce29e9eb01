"""MI355X-native CSA / HCA compressed-attention hot path.

The library (libsckv.so, hand-written HIP kernels for gfx950 behind a C ABI,
declared in include/sckv.h) exports csa_compress, csa_index_topk, csa_attend,
hca_compress and hca_attend; this package binds them for torch device tensors.
"""
from ._lib import (BF16, E4M3, F32, ROWS_CAUSAL, ROWS_DECODE, Pool, RowSpec, SckvError, abi_version,
                   attend_args, csa_attend, csa_compress, csa_index_score, csa_index_topk, csa_topk_select,
                   hca_attend, hca_compress, index_args, lib_path, load)

__all__ = ["BF16", "E4M3", "F32", "ROWS_CAUSAL", "ROWS_DECODE", "Pool", "RowSpec", "SckvError", "abi_version",
           "attend_args", "csa_attend", "csa_compress", "csa_index_score", "csa_index_topk", "csa_topk_select",
           "hca_attend", "hca_compress", "index_args", "lib_path", "load"]
