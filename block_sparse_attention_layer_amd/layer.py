"""One VMoBA attention layer as torch autograd functions over the C ABI.

papernotes 方法详解/整体框架: partition + block mean -> block selection -> attention on
the selected blocks.  The selection is computed in the forward and held constant in the
backward (it is not differentiated), so it runs outside the autograd function and the
function itself is the block-sparse attention over a fixed set of lists.  The full
attention of the warm-up steps (papernotes 损失函数/训练策略) is the dense kernel pair.
"""

from typing import Optional, Sequence, Tuple, Union

import torch

from .api import (Problem, Selection, vmoba_dense_attn_bwd, vmoba_dense_attn_fwd,
                  vmoba_partition_pool, vmoba_select, vmoba_sparse_attn_bwd,
                  vmoba_sparse_attn_fwd)


class VMoBAAttention(torch.autograd.Function):
    """Block-sparse attention over the lists of ``sel`` (CSR for O and dQ, CSC for dK/dV)."""

    @staticmethod
    def forward(ctx, q, k, v, problem, sel):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
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


class DenseAttention(torch.autograd.Function):
    """Full softmax attention over all L^2 pairs (the dense kernels)."""

    @staticmethod
    def forward(ctx, q, k, v, problem):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = vmoba_dense_attn_fwd(problem, q, k, v)
        ctx.problem = problem
        ctx.save_for_backward(q, k, v, o, lse)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = vmoba_dense_attn_bwd(ctx.problem, q, k, v, o, lse, do.contiguous())
        return dq, dk, dv, None


ListsLike = Union[Selection, Sequence[torch.Tensor]]


def as_selection(lists: ListsLike) -> Selection:
    """A Selection from a Selection or a (row_ptr, col_idx, col_ptr, row_idx) tuple."""
    if isinstance(lists, Selection):
        return lists
    row_ptr, col_idx, col_ptr, row_idx = lists
    return Selection(row_ptr=row_ptr, col_idx=col_idx, col_ptr=col_ptr, row_idx=row_idx,
                     head_stats=None)


def layer_problem(q, latent, layer_idx, block, grad_dtype=None) -> Problem:
    B, L, Hh, d = q.shape
    T, H, W = latent
    if L != T * H * W:
        raise ValueError(f"token count {L} != T*H*W = {T * H * W}")
    return Problem(B, Hh, d, T, H, W, layer_idx, tuple(block), q.dtype, grad_dtype)


def select_blocks(problem: Problem, q, k, *, tau: Optional[float] = 0.25,
                  mode: str = "threshold_global", topk: Optional[int] = None) -> Selection:
    """Pooling and block selection of one layer (no gradient flows through them)."""
    with torch.no_grad():
        qp, kp = vmoba_partition_pool(problem, q.detach().contiguous(),
                                      k.detach().contiguous())
        return vmoba_select(problem, qp, kp, tau, mode=mode, k=topk)


def vmoba_attention(q, k, v, *, latent, layer_idx, block, tau=0.25,
                    mode: str = "threshold_global", topk: Optional[int] = None,
                    selection: Optional[ListsLike] = None, return_selection=False):
    """q, k, v: [B, L, Hh, d] bf16 or fp32 on the GPU, L = T*H*W for latent (T, H, W).

    The layer's partition is picked by ``layer_idx mod 3`` (0: 1D, 1: 2D, 2: 3D) with
    block shape ``block``.  ``mode`` is one of the selection strategies (the default is
    the threshold over the whole head's pool); ``selection`` replaces the layer's own
    selection by caller lists.  Returns O (and the Selection with return_selection).
    """
    p = layer_problem(q, latent, layer_idx, block)
    sel = (as_selection(selection) if selection is not None
           else select_blocks(p, q, k, tau=tau, mode=mode, topk=topk))
    o = VMoBAAttention.apply(q, k, v, p, sel)
    return (o, sel) if return_selection else o


def full_attention(q, k, v, *, latent):
    """Dense softmax attention of q, k, v [B, L, Hh, d] with the library's dense kernels."""
    T, H, W = latent
    # the dense kernels use no partition; any valid one (one 1D block) describes the shape
    p = layer_problem(q, latent, 0, (T, H, W))
    return DenseAttention.apply(q, k, v, p)
