"""Seeded synthetic inputs for the VMoBA layer workloads.

This module holds shapes and random draws only — none of the method's
arithmetic.  The tests, the benchmark and the smoke check draw their inputs
here and hand the same tensors to the HIP library and to the CPU oracle.

The pages train and evaluate on Wan 2.1 1.3B with Koala-36M and VBench
(papernotes Table 1/Table 2; paperlayer §4.1).  Neither the weights nor the
data exist here, so seeded inputs of the pages' token counts stand in for them:
55,296 = 24*36*64 tokens for the 93x576x1024 training length and
75,600 = 21*45*80 for the 81x720x1280 (720p) length.

Recipe (per layer): draw order is the smooth field F, then eps_Q, eps_K, V and
(if a backward pass is needed) dO, all with one ``torch.Generator`` seeded by
``1000 * config_index + layer_in_cycle``.  F is N(0, 1) on a grid 4x coarser
in each of (T, H, W) (rounded up), trilinearly upsampled
(``align_corners=False``) per (batch, head, channel); then Q = F + 0.5 eps_Q and
K = F + 0.5 eps_K (one shared field, independent noise), V and dO i.i.d.
N(0, 1).  The ``tiny`` workload draws Q, K, V i.i.d. N(0, 1).  Draws are fp32
on the CPU and are then cast to the workload's dtype.
"""

from .configs import CONFIGS, CONFIG_ORDER, LayerSpec, config_layers
from .dit import PARAM_ORDER, make_dit_input, make_dit_params
from .inputs import make_layer_inputs, seed_for

__all__ = ["CONFIGS", "CONFIG_ORDER", "LayerSpec", "PARAM_ORDER", "config_layers",
           "make_dit_input", "make_dit_params", "make_layer_inputs", "seed_for"]
