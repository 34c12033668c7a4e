"""VMoBA block-sparse attention layer for AMD MI355X (gfx950).

The compute path is libvmoba.so (HIP kernels behind the C ABI of include/vmoba.h);
this package is its Python binding.
"""

from .api import (Problem, Selection, TokenSelection, vmoba_select_tokens,
                  vmoba_token_attn_bwd, vmoba_token_attn_fwd,
                  vmoba_dense_attn_bwd, vmoba_dense_attn_fwd,
                  vmoba_num_blocks, vmoba_partition_pool, vmoba_select,
                  vmoba_sparse_attn_bwd, vmoba_sparse_attn_bwd_delta,
                  vmoba_sparse_attn_bwd_noalloc,
                  vmoba_sparse_attn_bwd_dkdv, vmoba_sparse_attn_bwd_dq,
                  vmoba_sparse_attn_fwd, vmoba_validate,
                  vmoba_workspace_size)
from ._lib import VMoBAError, lib
from .layer import (DenseAttention, VMoBAAttention, as_selection, full_attention,
                    select_blocks, vmoba_attention)
from .dit import (LayerCycle, SyntheticDiT, SyntheticDiTBlock, full_attention_step,
                  num_full_steps)

__all__ = [
    "DenseAttention", "LayerCycle", "Problem", "Selection", "SyntheticDiT",
    "SyntheticDiTBlock", "TokenSelection", "VMoBAError", "VMoBAAttention", "as_selection", "full_attention",
    "full_attention_step", "lib", "num_full_steps", "select_blocks", "vmoba_attention",
    "vmoba_dense_attn_bwd", "vmoba_dense_attn_fwd", "vmoba_num_blocks",
    "vmoba_partition_pool", "vmoba_select", "vmoba_sparse_attn_bwd",
    "vmoba_sparse_attn_bwd_delta", "vmoba_sparse_attn_bwd_dkdv", "vmoba_sparse_attn_bwd_dq",
    "vmoba_sparse_attn_bwd_noalloc",
    "vmoba_sparse_attn_fwd", "vmoba_validate", "vmoba_workspace_size",
    "vmoba_select_tokens", "vmoba_token_attn_fwd", "vmoba_token_attn_bwd",
]
