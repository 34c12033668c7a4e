"""Oracle: block-mean pooling of Q and K (test infrastructure only).

papernotes, 关键设计 1: the keys, rearranged into the blocks of the layer's
partition, are averaged to a block tensor B = mean(K').  Reading taken: the
queries are pooled with the same partition (the pages pool only K; with
query blocks the block score is the mean over a query block of the
token-level scores q_i b_i^T of papernotes 关键设计 2, by linearity).
"""

import numpy as np


def block_means(x, members):
    """Mean over each block's tokens.

    x:       ``[B, L, Hh, d]`` array (any float dtype; upcast to fp64)
    members: ``[N_b, S]`` token table from :func:`oracle.partition.block_members`
    returns  ``[B, Hh, N_b, d]`` fp64
    """
    x = np.asarray(x, dtype=np.float64)
    B, L, Hh, d = x.shape
    nb, S = members.shape
    out = np.empty((B, Hh, nb, d), dtype=np.float64)
    for i in range(nb):
        acc = np.zeros((B, Hh, d), dtype=np.float64)
        for x_tok in members[i]:
            acc += x[:, x_tok, :, :]
        out[:, :, i, :] = acc / S
    return out
