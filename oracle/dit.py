"""Oracle: the VMoBA attention inside one DiT block, fp64 on the CPU (test
infrastructure only).

papernotes 方法详解/整体框架: the layer replaces full attention inside the video
diffusion transformer and keeps its input/output contract (heads computed separately
and concatenated); papernotes 关键设计 1 picks the partition of layer l by l mod 3;
papernotes 损失函数/训练策略 keeps full attention for the first denoising steps.

The block around the attention is the usual pre-norm DiT block (the pages do not
describe it; it is the plainest host for the layer):

    h = LN(x);  q, k, v = h Wq^T + bq, h Wk^T + bk, h Wv^T + bv   (split into heads:
                                   head j = channels j*d .. j*d + d - 1)
    x = x + Attn(q, k, v) Wo^T + bo
    x = x + GELU_tanh(LN(x) W1^T + b1) W2^T + b2

with LN the layer norm without affine parameters (eps 1e-6).  Attn is the oracle's
masked attention over the layer's own selection (pool -> select on the block's q and
k, held constant in the backward), or over all pairs for a full-attention step.  The
norm, the products and the GELU are torch fp64 library routines and the gradients come
from torch autograd; the attention's forward and backward are the oracle's own.
"""

import numpy as np
import torch
import torch.nn.functional as F

from .attention import sparse_attention_bwd, sparse_attention_fwd
from .partition import block_members, check_partition
from .pooling import block_means
from .selection import select_all_heads


class _OracleAttention(torch.autograd.Function):
    """Masked attention of the oracle as a torch function (mask constant)."""

    @staticmethod
    def forward(ctx, q, k, v, members, mask):
        qn, kn, vn = (t.detach().numpy() for t in (q, k, v))
        o, lse = sparse_attention_fwd(qn, kn, vn, members, mask)
        ctx.save = (qn, kn, vn, o, lse, members, mask)
        return torch.from_numpy(o)

    @staticmethod
    def backward(ctx, do):
        qn, kn, vn, o, lse, members, mask = ctx.save
        dq, dk, dv = sparse_attention_bwd(qn, kn, vn, o, lse, do.detach().numpy(),
                                          members, mask)
        return torch.from_numpy(dq), torch.from_numpy(dk), torch.from_numpy(dv), None, None


def layer_selection(q, k, latent, layer_idx, block, tau=0.25, mode="threshold_global",
                    k_top=None):
    """(members, mask, shat, stats) of one layer from its q, k [B, L, Hh, d]."""
    T, H, W = latent
    check_partition(T, H, W, layer_idx, block)
    members = block_members(T, H, W, block)
    qn = q.detach().numpy() if torch.is_tensor(q) else np.asarray(q, np.float64)
    kn = k.detach().numpy() if torch.is_tensor(k) else np.asarray(k, np.float64)
    mask, shat, stats = select_all_heads(block_means(qn, members), block_means(kn, members),
                                         tau, mode=mode, k=k_top)
    return members, mask, shat, stats


def dit_block(x, params, latent, heads, layer_idx, block, *, tau=0.25, full=False,
              mask=None, mode="threshold_global", k_top=None):
    """One block.  x: fp64 tensor [B, L, dim]; params: dict of fp64 tensors
    (wq, bq, wk, bk, wv, bv, wo, bo, w1, b1, w2, b2; Linear layout [out, in]).

    ``mask`` ([B, Hh, N_b, N_b] bool) holds the selection fixed; by default the block
    selects from its own q and k.  Returns (y, info) with info = dict(members, mask,
    shat, stats) of the attention used (shat/stats None when given or full).
    """
    B, L, dim = x.shape
    d = dim // heads
    P = params
    h = F.layer_norm(x, (dim,), eps=1e-6)
    q = (h @ P["wq"].T + P["bq"]).reshape(B, L, heads, d)
    k = (h @ P["wk"].T + P["bk"]).reshape(B, L, heads, d)
    v = (h @ P["wv"].T + P["bv"]).reshape(B, L, heads, d)
    info = dict(shat=None, stats=None)
    if full:
        # every token attends to every token: one block of all tokens, selected
        members = np.arange(L)[None, :]
        mask = np.ones((B, heads, 1, 1), dtype=bool)
    elif mask is None:
        members, mask, info["shat"], info["stats"] = layer_selection(
            q, k, latent, layer_idx, block, tau, mode, k_top)
    else:
        T, H, W = latent
        check_partition(T, H, W, layer_idx, block)
        members = block_members(T, H, W, block)
    info.update(members=members, mask=mask)
    a = _OracleAttention.apply(q, k, v, members, mask)
    x = x + a.reshape(B, L, dim) @ P["wo"].T + P["bo"]
    h = F.layer_norm(x, (dim,), eps=1e-6)
    y = x + F.gelu(h @ P["w1"].T + P["b1"], approximate="tanh") @ P["w2"].T + P["b2"]
    return y, info


def full_attention_step(step, num_steps, warmup=0.25):
    """Whether denoising step ``step`` (0-based, in run order) of ``num_steps`` keeps full
    attention: the first 25 % of the steps do.  Reading: a step is in the first 25 % when
    step < 0.25 * num_steps, so the count of full steps rounds up (13 of 50)."""
    return step < warmup * num_steps


def dit_stack(x, params, latent, heads, blocks, *, tau=0.25, step=None, num_steps=None,
              warmup=0.25, masks=None):
    """Layers 0 .. n-1 with block shapes blocks[l % 3] (1D, 2D, 3D), and the warm-up rule.
    Returns (y, infos)."""
    full = step is not None and full_attention_step(step, num_steps, warmup)
    infos = []
    for layer, p in enumerate(params):
        x, info = dit_block(x, p, latent, heads, layer, blocks[layer % 3], tau=tau,
                            full=full, mask=None if masks is None else masks[layer])
        infos.append(info)
    return x, infos
