"""Pins of the oracle's partition (CPU only).

papernotes 关键设计 1 / paperlayer §3.2: l mod 3 -> 1D temporal, 2D spatial
(same spatial position across all frames), 3D local box.
"""

import itertools

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def test_mode_table():
    # l mod 3 = 0 -> 1D, 1 -> 2D, 2 -> 3D (papernotes 关键设计 1), cycling.
    expect = {0: oracle.MODE_1D, 1: oracle.MODE_2D, 2: oracle.MODE_3D,
              3: oracle.MODE_1D, 4: oracle.MODE_2D, 5: oracle.MODE_3D,
              29: oracle.MODE_3D}
    for l, m in expect.items():
        assert oracle.partition_mode(l) == m
    with pytest.raises(ValueError):
        oracle.partition_mode(-1)


@pytest.mark.parametrize("args", [
    (4, 8, 8, 2, (3, 4, 4)),      # 3 does not divide T=4
    (4, 8, 8, 0, (1, 4, 8)),      # 1D block must hold whole frames
    (4, 8, 8, 1, (2, 4, 4)),      # 2D block must span all frames
    (4, 8, 8, 2, (0, 4, 4)),
])
def test_rejects_bad_partitions(args):
    with pytest.raises(ValueError):
        oracle.check_partition(*args)


def _coords(tok, H, W):
    t, rem = np.divmod(tok, H * W)
    h, w = np.divmod(rem, W)
    return t, h, w


@pytest.mark.parametrize("T,H,W,layer,block", [
    (4, 8, 8, 2, (2, 4, 4)),
    (6, 4, 10, 0, (2, 4, 10)),
    (6, 4, 10, 1, (6, 2, 5)),
    (5, 3, 7, 2, (5, 3, 7)),
    (3, 6, 4, 2, (1, 1, 1)),
])
def test_blocks_are_boxes_covering_every_token_once(T, H, W, layer, block):
    mode = oracle.check_partition(T, H, W, layer, block)
    mem = oracle.block_members(T, H, W, block)
    L = T * H * W
    bt, bh, bw = block
    # every token in exactly one block; equal block sizes
    assert sorted(mem.reshape(-1).tolist()) == list(range(L))
    assert mem.shape == (oracle.num_blocks(T, H, W, block), bt * bh * bw)
    for row in mem:
        t, h, w = _coords(row, H, W)
        # the block is an aligned box of the block shape ...
        box = set(itertools.product(range(t.min(), t.min() + bt),
                                    range(h.min(), h.min() + bh),
                                    range(w.min(), w.min() + bw)))
        assert set(zip(t.tolist(), h.tolist(), w.tolist())) == box
        assert t.min() % bt == 0 and h.min() % bh == 0 and w.min() % bw == 0
        # ... listed in row-major (t, h, w) order
        key = list(zip(t.tolist(), h.tolist(), w.tolist()))
        assert key == sorted(key)
        if mode == oracle.MODE_1D:   # whole frames
            assert set(h.tolist()) == set(range(H))
            assert set(w.tolist()) == set(range(W))
        if mode == oracle.MODE_2D:   # every frame at the same spatial patch
            assert set(t.tolist()) == set(range(T))
    # block ids are row-major over the block grid
    first = [tuple(int(c) for c in _coords(row[0], H, W)) for row in mem]
    assert first == sorted(first)
    blk = oracle.block_of_token(mem, L)
    for i, row in enumerate(mem):
        assert (blk[row] == i).all()


def test_workload_block_counts():
    # block counts of the five workloads (from their latent and block shapes)
    cases = {((4, 8, 8), (2, 4, 4)): 8, ((21, 30, 52), (1, 30, 52)): 21,
             ((21, 30, 52), (21, 6, 4)): 65, ((24, 36, 64), (4, 6, 8)): 288,
             ((21, 45, 80), (1, 45, 80)): 21, ((21, 45, 80), (21, 9, 8)): 50,
             ((21, 45, 80), (3, 9, 8)): 350}
    for (lat, blk), nb in cases.items():
        assert oracle.num_blocks(*lat, blk) == nb
