"""One VMoBA attention layer as a torch autograd function over the C ABI.

papernotes 方法详解/整体框架: partition + block mean -> global block selection with the
threshold tau -> attention on the selected blocks.  The selection is computed in the
forward and held constant in the backward (it is not differentiated).
"""

import torch

from .api import (Problem, vmoba_partition_pool, vmoba_select, vmoba_sparse_attn_bwd,
                  vmoba_sparse_attn_fwd)


class VMoBAAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, problem, tau):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        qp, kp = vmoba_partition_pool(problem, q, k)
        sel = vmoba_select(problem, qp, kp, tau)
        o, lse = vmoba_sparse_attn_fwd(problem, q, k, v, sel.row_ptr, sel.col_idx)
        ctx.problem = problem
        ctx.sel = sel
        ctx.save_for_backward(q, k, v, o, lse)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        s = ctx.sel
        dq, dk, dv = vmoba_sparse_attn_bwd(ctx.problem, q, k, v, o, lse, do.contiguous(),
                                           s.row_ptr, s.col_idx, s.col_ptr, s.row_idx)
        return dq, dk, dv, None, None


def vmoba_attention(q, k, v, *, latent, layer_idx, block, tau=0.25):
    """q, k, v: [B, L, Hh, d] bf16 or fp32 on the GPU, L = T*H*W for latent (T, H, W)."""
    B, L, Hh, d = q.shape
    T, H, W = latent
    p = Problem(B, Hh, d, T, H, W, layer_idx, tuple(block), q.dtype)
    return VMoBAAttention.apply(q, k, v, p, float(tau))
