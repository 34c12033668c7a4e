"""VMoBA block-sparse attention layer for AMD MI355X (gfx950).

The compute path is libvmoba.so (HIP kernels behind the C ABI of include/vmoba.h);
this package is its Python binding.
"""

from .api import (Problem, Selection, vmoba_dense_attn_bwd, vmoba_dense_attn_fwd,
                  vmoba_num_blocks, vmoba_partition_pool, vmoba_select,
                  vmoba_sparse_attn_bwd, vmoba_sparse_attn_bwd_delta,
                  vmoba_sparse_attn_bwd_dkdv, vmoba_sparse_attn_bwd_dq,
                  vmoba_sparse_attn_fwd, vmoba_validate,
                  vmoba_workspace_size)
from ._lib import VMoBAError, lib
from .layer import VMoBAAttention, vmoba_attention

__all__ = [
    "Problem", "Selection", "VMoBAError", "VMoBAAttention", "lib", "vmoba_attention",
    "vmoba_dense_attn_bwd", "vmoba_dense_attn_fwd", "vmoba_num_blocks",
    "vmoba_partition_pool", "vmoba_select", "vmoba_sparse_attn_bwd",
    "vmoba_sparse_attn_bwd_delta", "vmoba_sparse_attn_bwd_dkdv", "vmoba_sparse_attn_bwd_dq",
    "vmoba_sparse_attn_fwd", "vmoba_validate", "vmoba_workspace_size",
]
