"""Host logic of the DiT integration (CPU only): the layer cycle and the warm-up switch.

The warm-up count is checked against the oracle's reading of the rule (the first 25 %
of the denoising steps keep full attention: step < 0.25 * num_steps).
"""

import pytest

from oracle import dit as odit
from oracle import partition_mode, MODE_1D, MODE_2D, MODE_3D
from block_sparse_attention_layer_amd import LayerCycle, full_attention_step, num_full_steps


def test_warmup_switch_agrees_with_oracle_reading():
    for n in range(1, 101):
        for s in range(n):
            assert full_attention_step(s, n) == odit.full_attention_step(s, n), (s, n)
    assert num_full_steps(50) == 13 and num_full_steps(40) == 10
    assert num_full_steps(50, warmup=0.0) == 0 and num_full_steps(7, warmup=1.0) == 7


def test_warmup_switch_rejects_bad_arguments():
    with pytest.raises(ValueError):
        full_attention_step(4, 4)
    with pytest.raises(ValueError):
        full_attention_step(-1, 4)
    with pytest.raises(ValueError):
        full_attention_step(0, 4, warmup=1.5)


def test_layer_cycle_follows_partition_mode():
    cyc = LayerCycle((24, 36, 64), (3, 36, 64), (24, 6, 8), (8, 12, 8))   # 8-48-72
    names = {MODE_1D: "1d", MODE_2D: "2d", MODE_3D: "3d"}
    for layer in range(12):
        assert cyc.mode(layer) == names[partition_mode(layer)]
    assert [cyc.num_blocks(l) for l in range(6)] == [8, 48, 72, 8, 48, 72]
    assert cyc.block(5) == (8, 12, 8)


@pytest.mark.parametrize("blocks", [
    ((3, 6, 64), (24, 6, 8), (8, 12, 8)),    # 1D must span whole frames
    ((3, 36, 64), (12, 6, 8), (8, 12, 8)),   # 2D must span all frames
    ((3, 36, 64), (24, 6, 8), (5, 12, 8)),   # 3D must divide the latent
])
def test_layer_cycle_rejects_invalid_partitions(blocks):
    with pytest.raises(ValueError):
        LayerCycle((24, 36, 64), *blocks)
