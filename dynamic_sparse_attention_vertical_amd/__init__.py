"""MI355X-native vertical-slash dynamic sparse prefill attention.

The computation lives in libmsa.so (hand-written HIP kernels for gfx950 behind
the C ABI declared in include/msa.h); this package is a thin ctypes binding
over it.  PyTorch provides device memory and streams only.
"""

from .msa import (MsaError, IndexTensors, Problem, alloc_index, build_index, decode_sparse,
                  decode_sparse_workspace_bytes, dense_prefill, build_index_varlen, dense_prefill_varlen,
                  estimate_bs_varlen, estimate_vs_varlen, sparse_prefill_varlen,
                  estimate_vs_varlen_workspace_bytes, sparse_prefill_varlen_workspace_bytes, varlen,
                  estimate_bs, estimate_vs, estimate_vs_noalloc, estimate_vs_workspace_bytes, index_caps, lib_path, load,
                  problem, sparse_prefill, sparse_prefill_fused, sparse_prefill_fused_workspace_bytes,
                  sparse_prefill_workspace_bytes,
                  sparse_walk_marks)
from .layer import (vertical_slash_layer, mixed_layer, vertical_slash_sparse_attention, block_sparse_attention,
                    streaming_forward)
from .graphs import StepGraph, decode_graph, layer_graph

__all__ = ["MsaError", "IndexTensors", "Problem", "alloc_index", "build_index", "decode_sparse",
           "decode_sparse_workspace_bytes", "dense_prefill", "build_index_varlen", "dense_prefill_varlen",
           "estimate_bs_varlen", "estimate_vs_varlen", "sparse_prefill_varlen",
           "estimate_vs_varlen_workspace_bytes", "sparse_prefill_varlen_workspace_bytes", "varlen",
           "estimate_bs", "estimate_vs", "estimate_vs_noalloc", "estimate_vs_workspace_bytes", "index_caps", "lib_path",
           "load", "problem", "sparse_prefill", "sparse_prefill_fused", "sparse_prefill_fused_workspace_bytes",
           "sparse_prefill_workspace_bytes",
           "sparse_walk_marks", "vertical_slash_layer", "mixed_layer",
           "vertical_slash_sparse_attention", "block_sparse_attention", "streaming_forward",
           "StepGraph", "decode_graph", "layer_graph"]
