"""Oracle: one whole VMoBA layer, in the pages' order (test infrastructure only).

papernotes 方法详解/整体框架 flowchart: partition + block mean -> global block
selection -> threshold k -> sparse attention with the heads concatenated.
"""

from .partition import check_partition, block_members, block_of_token
from .pooling import block_means
from .selection import select_all_heads
from .attention import sparse_attention_fwd, sparse_attention_bwd


def oracle_layer(q, k, v, T, H, W, layer_idx, block, tau, do=None):
    """Run pool -> select -> attention (and backward if ``do`` is given) in fp64.

    Returns a dict with members, q_pool, k_pool, mask, shat, stats, o, lse and,
    when ``do`` is given, dq, dk, dv.
    """
    check_partition(T, H, W, layer_idx, block)
    members = block_members(T, H, W, block)
    L = T * H * W
    qp = block_means(q, members)
    kp = block_means(k, members)
    mask, shat, stats = select_all_heads(qp, kp, tau)
    o, lse = sparse_attention_fwd(q, k, v, members, mask)
    out = {"members": members, "block_of_tok": block_of_token(members, L),
           "q_pool": qp, "k_pool": kp, "mask": mask, "shat": shat,
           "stats": stats, "o": o, "lse": lse}
    if do is not None:
        dq, dk, dv = sparse_attention_bwd(q, k, v, o, lse, do, members, mask)
        out.update(dq=dq, dk=dk, dv=dv)
    return out

