"""CPU oracle for the VMoBA attention layer — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, fp64 NumPy implementation of what one VMoBA
attention layer computes.  It exists to check the HIP path; it is not part of
the product.  Only the test-suite, the smoke check of the build entry point and
the ``cpu_baseline`` leg of the benchmark may import it.  It shares no code,
table or constant with the HIP library, and it imports nothing from the
product package.

Sources followed (two web pages on the method; cited below by short name):

* ``papernotes`` — papernotes.org reading notes "VMoBA: Mixture-of-Block
  Attention for Video Diffusion Models" (ICLR 2026): sections 方法详解/整体框架
  (overall pipeline), 关键设计 1 (layer-wise recurrent 1D-2D-3D partition and
  the block mean), 关键设计 2 (global block selection), 关键设计 3 (threshold
  equation for the dynamic block count).
* ``paperlayer`` — paperlayer.ai digest of arXiv 2506.23858: §3.1 (overview,
  Fig. 2), §3.2 (partition, Fig. 3), §3.3 (global selection, Fig. 4), §3.4
  (threshold selection, Fig. 5).

Where the pages leave a step open the reading taken is stated next to the code
that takes it.  Modules:

* :mod:`oracle.partition` — mode ``l mod 3`` and the block membership table.
* :mod:`oracle.pooling` — block means of Q and K.
* :mod:`oracle.selection` — block scores, per-head softmax normalisation and
  the cumulative-mass threshold with the forced diagonal; the ablation's other
  strategies (top-k + global, threshold + local, top-k + local; paperlayer §4.4,
  Table 3).
* :mod:`oracle.attention` — masked softmax attention forward and backward
  (literal dense form, block-sparse form and sampled rows).
* :mod:`oracle.tokens` — the token-granular query pool (every query token against every
  key block) and the attention under its per-token selection.
* :mod:`oracle.dit` — the layer inside a DiT block and stack (projections, MLP, the
  1D/2D/3D layer cycle, the full-attention warm-up).

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, library routines, invariants and brute force on tiny inputs.  The pages
print no worked numeric example, so no value on the pages pins any number.
"""

from .partition import (
    MODE_1D, MODE_2D, MODE_3D, partition_mode, check_partition, block_members,
    block_of_token, num_blocks,
)
from .pooling import block_means
from .selection import (
    block_scores, normalise_per_head, threshold_select, select_all_heads,
    mask_to_csr, mask_to_csc, topk_select, normalise_per_row, local_select,
    SELECTION_MODES,
)
from .attention import (
    dense_masked_attention_fwd, dense_masked_attention_bwd, token_mask,
    sparse_attention_fwd, sparse_attention_bwd, sampled_query_rows,
    sampled_key_block_grads,
)
from .layer import oracle_layer
from .tokens import (
    token_scores, normalise_token_pool, token_select, select_tokens_all_heads,
    union_block_mask, token_level_mask, token_attention_fwd, token_attention_bwd,
    sampled_token_rows,
)

__all__ = [
    "MODE_1D", "MODE_2D", "MODE_3D", "partition_mode", "check_partition",
    "block_members", "block_of_token", "num_blocks", "block_means",
    "block_scores", "normalise_per_head", "threshold_select",
    "select_all_heads", "mask_to_csr", "mask_to_csc", "topk_select",
    "normalise_per_row", "local_select", "SELECTION_MODES",
    "dense_masked_attention_fwd", "dense_masked_attention_bwd", "token_mask",
    "sparse_attention_fwd", "sparse_attention_bwd", "sampled_query_rows",
    "sampled_key_block_grads", "oracle_layer", "token_scores", "normalise_token_pool",
    "token_select", "select_tokens_all_heads", "union_block_mask", "token_level_mask",
    "token_attention_fwd", "token_attention_bwd", "sampled_token_rows",
]
