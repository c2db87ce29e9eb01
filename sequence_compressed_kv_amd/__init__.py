"""MI355X-native CSA / HCA compressed-attention hot path.

The library (libsckv.so, hand-written HIP kernels for gfx950 behind a C ABI,
declared in include/sckv.h) exports csa_compress, csa_index_topk, csa_attend,
hca_compress and hca_attend (plus the decode appends csa_append / hca_append and
the decode projections layer_queries / layer_streams / layer_inputs /
layer_output); this package binds them for torch device tensors.
"""
from ._lib import (BF16, E4M3, F32, LAYOUT_KEY_TILES, LAYOUT_ROWS, MXFP4, ROWS_CAUSAL, ROWS_DECODE, Append,
                   Mxfp4Keys, Pool, RowSpec, SckvError, abi_version, attend_args, csa_append, csa_attend, csa_compress, csa_index_score,
                   csa_index_topk, csa_index_topk_noalloc, csa_topk_select, from_key_tiles, hca_append, hca_attend, hca_compress, index_args,
                   key_tiles_empty, layer_inputs, layer_output, layer_queries, layer_streams, lib_path, load,
                   mxfp4_pack, mxfp4_unpack, output_args, query_args, stream_args, to_key_tiles)

__all__ = ["BF16", "E4M3", "F32", "LAYOUT_KEY_TILES", "LAYOUT_ROWS", "MXFP4", "ROWS_CAUSAL", "ROWS_DECODE", "Append",
           "Mxfp4Keys", "Pool", "RowSpec", "SckvError", "abi_version", "attend_args", "csa_append", "csa_attend", "csa_compress",
           "csa_index_score", "csa_index_topk", "csa_index_topk_noalloc", "csa_topk_select", "from_key_tiles", "hca_append", "hca_attend",
           "hca_compress", "index_args", "key_tiles_empty", "layer_inputs", "layer_output", "layer_queries",
           "layer_streams", "lib_path", "load", "mxfp4_pack", "mxfp4_unpack", "output_args", "query_args", "stream_args", "to_key_tiles"]
