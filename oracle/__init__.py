"""CPU oracle for vertical-slash dynamic sparse prefill attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product path (the
HIP library and its Python binding) never calls it, and it never calls the
product path: the two share no code, tables or helpers.

What it computes, in float64 from the exact input values, written as the plain
definitions (no blocking, fusion or reordering beyond what the definitions
state):

  estimate.estimate_vs     online vertical/slash score estimate from the last
                           queries ("MInference 1.0 README", section "TL;DR":
                           the sparse index is approximated online per head;
                           talk slides "System-Algorithm Co-design", slide
                           "MInference", step 2 "Online Estimation of Sparsity
                           Indices"; column index and slash index, slide
                           "Dynamic sparsity in attention").
  estimate.top_k_indices   exact top-k with ties going to the lower index.
  estimate.block_sparse_select
                           mean-pooled block scores, top-k key blocks per query
                           block (block-sparse pattern, same slides, patterns
                           list; "MInference 1.0 README", kernel-only usage
                           block_sparse_attention(q, k, v, topk)).
  index.build_index        selected diagonals -> per-query-block lists of
                           64-wide key blocks plus leftover vertical columns
                           (plain C helper, see csrc/index_ref.c).
  index.exact_union_mask   M_x: the selected columns and diagonals themselves
  index.exact_union_rows   (the vertical-slash pattern as the talk slides
                           draw it, slide "Dynamic sparsity in attention");
                           the second gives given rows only.
  decode.*                 one decode query row per head over a key cache:
                           scores, attention over the top-k keys (or a given
                           set) and the kept share of the dense attention mass
                           (talk slides, slide "Dynamic sparsity in attention",
                           decoding panel).
  attention.*              softmax attention restricted to an explicit boolean
                           mask (dense causal when every column and diagonal is
                           selected); attention_recall, the share of each
                           row's dense attention that a mask keeps.

Pins that tie each function to something other than itself live in
tests/test_oracle_pins.py.
"""

from .estimate import estimate_vs, top_k_indices, block_sparse_select, block_scores
from .index import (build_index, a_shape_sets, index_mask, exact_union_mask, exact_union_rows,
                    block_key_sets, IndexArrays)
from .attention import (attention_with_mask, masked_attention_blocks, exact_attention_blocks,
                        dense_attention_blocks, dense_attention, attention_recall)
from .decode import decode_scores, decode_sparse_attention

__all__ = [
    "estimate_vs", "top_k_indices", "block_sparse_select", "block_scores",
    "build_index", "a_shape_sets", "index_mask", "exact_union_mask", "exact_union_rows", "block_key_sets",
    "IndexArrays",
    "attention_with_mask", "masked_attention_blocks", "exact_attention_blocks", "dense_attention_blocks",
    "dense_attention", "attention_recall", "decode_scores", "decode_sparse_attention",
]
