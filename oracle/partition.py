"""Oracle: the layer-wise recurrent 1D-2D-3D partition (test infrastructure only).

papernotes, 关键设计 1; paperlayer §3.2 (Fig. 3).  Layer ``l`` partitions the
(T, H, W) video latent by ``l mod 3``:

* 0 -> 1D temporal blocks: a run of adjacent whole frames;
* 1 -> 2D spatial blocks: one spatial patch taken across *all* frames;
* 2 -> 3D spatio-temporal blocks: a local (t, h, w) box.

Readings taken where the pages are silent:

* layers are numbered from 0;
* an extent that the block shape does not divide is rejected;
* blocks are numbered row-major over the block grid (t outer, w inner) and the
  tokens inside a block are listed row-major over (dt, dh, dw).  Only the
  summation order of the block means and the index used to break exact ties
  depend on this choice.

Tokens are flattened frame-first: token (t, h, w) has index (t*H + h)*W + w.
"""

import numpy as np

MODE_1D, MODE_2D, MODE_3D = 0, 1, 2


def partition_mode(layer_idx):
    """Partition mode of layer ``layer_idx`` (papernotes 关键设计 1: l mod 3)."""
    if layer_idx < 0:
        raise ValueError("layer index must be >= 0")
    return layer_idx % 3


def check_partition(T, H, W, layer_idx, block):
    """Reject a block shape that is not a partition of the stated mode.

    1D blocks hold whole frames (b_h, b_w) = (H, W); 2D blocks hold every frame
    (b_t = T); 3D blocks may be any box.  Each extent must divide its axis.
    """
    bt, bh, bw = block
    if min(T, H, W, bt, bh, bw) <= 0:
        raise ValueError("extents and block sizes must be positive")
    if T % bt or H % bh or W % bw:
        raise ValueError("block shape must divide the latent (T, H, W)")
    mode = partition_mode(layer_idx)
    if mode == MODE_1D and (bh, bw) != (H, W):
        raise ValueError("a 1D (temporal) block holds whole frames")
    if mode == MODE_2D and bt != T:
        raise ValueError("a 2D (spatial) block spans all frames")
    return mode


def num_blocks(T, H, W, block):
    bt, bh, bw = block
    return (T // bt) * (H // bh) * (W // bw)


def block_members(T, H, W, block):
    """Token indices of every block, ``[N_b, S]`` int64, by explicit loops.

    Row ``i`` lists the tokens of block ``i`` in within-block row-major order.
    """
    bt, bh, bw = block
    nt, nh, nw = T // bt, H // bh, W // bw
    S = bt * bh * bw
    out = np.empty((nt * nh * nw, S), dtype=np.int64)
    i = 0
    for it in range(nt):
        for ih in range(nh):
            for iw in range(nw):
                r = 0
                for dt in range(bt):
                    t = it * bt + dt
                    for dh in range(bh):
                        h = ih * bh + dh
                        for dw in range(bw):
                            w = iw * bw + dw
                            out[i, r] = (t * H + h) * W + w
                            r += 1
                i += 1
    return out


def block_of_token(members, L):
    """Inverse of :func:`block_members`: block id of each of the ``L`` tokens."""
    blk = np.full(L, -1, dtype=np.int64)
    for i in range(members.shape[0]):
        blk[members[i]] = i
    return blk
