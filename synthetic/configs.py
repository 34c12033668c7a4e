"""The workloads: shapes, partitions, thresholds and passes.

Every workload has batch 1.  Block shapes follow the layer-cycled partition
(papernotes 关键设计 1): layer index l picks 1D (l mod 3 = 0), 2D (1) or 3D (2).
"""

from dataclasses import dataclass
from typing import Tuple


@dataclass(frozen=True)
class LayerSpec:
    layer_idx: int
    block: Tuple[int, int, int]


CONFIG_ORDER = ["tiny", "l1d_32k", "l2d_32k", "l3d_55k", "cycle_76k", "blocks_55k",
                "blocks_46k", "blocks_11k"]

CONFIGS = {
    # 256 tokens, fp32, 2 heads of 64, 3D blocks (2,4,4): 8 blocks of 32 tokens.
    "tiny": dict(batch=1, heads=2, head_dim=64, T=4, H=8, W=8,
                 layers=(LayerSpec(2, (2, 4, 4)),), taus=(0.25,),
                 dtype="fp32", backward=False, field="iid"),
    # 32,760 tokens, one latent frame per 1D block: 21 blocks of 1,560 tokens.
    "l1d_32k": dict(batch=1, heads=12, head_dim=128, T=21, H=30, W=52,
                    layers=(LayerSpec(0, (1, 30, 52)),), taus=(0.25,),
                    dtype="bf16", backward=False, field="smooth"),
    # 32,760 tokens, 6x4 spatial patches across all 21 frames: 65 blocks of 504.
    "l2d_32k": dict(batch=1, heads=12, head_dim=128, T=21, H=30, W=52,
                    layers=(LayerSpec(1, (21, 6, 4)),), taus=(0.25,),
                    dtype="bf16", backward=True, field="smooth"),
    # 55,296 tokens (93x576x1024 training length), 3D (4,6,8): 288 blocks of 192.
    "l3d_55k": dict(batch=1, heads=12, head_dim=128, T=24, H=36, W=64,
                    layers=(LayerSpec(2, (4, 6, 8)),), taus=(0.25,),
                    dtype="bf16", backward=True, field="smooth"),
    # 75,600 tokens (81x720x1280), one 1D/2D/3D cycle, tau swept.
    "cycle_76k": dict(batch=1, heads=12, head_dim=128, T=21, H=45, W=80,
                      layers=(LayerSpec(0, (1, 45, 80)), LayerSpec(1, (21, 9, 8)),
                              LayerSpec(2, (3, 9, 8))),
                      taus=(0.15, 0.25, 0.5), dtype="bf16", backward=True,
                      field="smooth"),
    # The pages' default block counts "8-48-72" for 1D/2D/3D (papernotes 训练策略, paperlayer
    # §4.4) on the 55,296-token latent: 1D blocks of 3 frames (8 blocks of 6,912 tokens),
    # 2D patches of 6x8 across all frames (48 of 1,152), and 3D blocks (8,12,8) (72 of 768;
    # the pages give no 3D shape, this is one of the factorisations into 72).
    "blocks_55k": dict(batch=1, heads=12, head_dim=128, T=24, H=36, W=64,
                       layers=(LayerSpec(0, (3, 36, 64)), LayerSpec(1, (24, 6, 8)),
                               LayerSpec(2, (8, 12, 8))),
                       taus=(0.25,), dtype="bf16", backward=True, field="smooth"),
    # The pre-training setting "10-48-60" of paperlayer App. C (Table 6): 1D/2D/3D block
    # counts 10, 48 and 60 at 46K and 11K tokens, tau 0.25.  The pages give no latent shape
    # for either length; these are factorisations with a frame count divisible by 10.
    # 46,080 tokens = 20x36x64: 1D blocks of 2 frames (10 of 4,608), 2D patches of 6x8
    # across all frames (48 of 960), 3D blocks (4,12,16) (5x3x4 = 60 of 768).
    "blocks_46k": dict(batch=1, heads=12, head_dim=128, T=20, H=36, W=64,
                       layers=(LayerSpec(0, (2, 36, 64)), LayerSpec(1, (20, 6, 8)),
                               LayerSpec(2, (4, 12, 16))),
                       taus=(0.25,), dtype="bf16", backward=True, field="smooth"),
    # 11,520 tokens = 10x24x48: 1D blocks of one frame (10 of 1,152), 2D patches of 4x6
    # across all frames (48 of 240), 3D blocks (2,8,12) (5x3x4 = 60 of 192).
    "blocks_11k": dict(batch=1, heads=12, head_dim=128, T=10, H=24, W=48,
                       layers=(LayerSpec(0, (1, 24, 48)), LayerSpec(1, (10, 4, 6)),
                               LayerSpec(2, (2, 8, 12))),
                       taus=(0.25,), dtype="bf16", backward=True, field="smooth"),
}


def config_layers(name):
    """(layer_in_cycle, LayerSpec) pairs of a workload."""
    return list(enumerate(CONFIGS[name]["layers"]))
