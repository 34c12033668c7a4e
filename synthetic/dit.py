"""Seeded synthetic weights and activations for a small DiT stack (random draws only).

The pages train Wan 2.1 1.3B (papernotes 损失函数/训练策略); its weights are not
available, so each block gets random weights of the same structure: q, k, v and output
projections dim -> dim with bias, and a two-layer MLP dim -> hidden -> dim with bias.
Weights are N(0, 1/fan_in), biases N(0, 0.02^2), all fp32 on the CPU from one
``torch.Generator``; block l draws with seed ``seed + l`` in the order
wq, bq, wk, bk, wv, bv, wo, bo, w1, b1, w2, b2.

The block input is a smooth field over the latent plus noise (the recipe of the layer
inputs: N(0, 1) on a grid 4x coarser in each of T, H, W, trilinearly upsampled, plus
0.5 N(0, 1)), so that the projected queries and keys carry the spatio-temporal
locality the block selection works on; the output cotangent is i.i.d. N(0, 1).
"""

import math

import torch
import torch.nn.functional as F

PARAM_ORDER = ("wq", "bq", "wk", "bk", "wv", "bv", "wo", "bo", "w1", "b1", "w2", "b2")


def make_dit_params(dim, mlp_hidden, num_layers, seed=7000):
    """List (one dict per block) of fp32 CPU weights; Linear layout [out, in]."""
    shapes = {"wq": (dim, dim), "bq": (dim,), "wk": (dim, dim), "bk": (dim,),
              "wv": (dim, dim), "bv": (dim,), "wo": (dim, dim), "bo": (dim,),
              "w1": (mlp_hidden, dim), "b1": (mlp_hidden,), "w2": (dim, mlp_hidden),
              "b2": (dim,)}
    out = []
    for layer in range(num_layers):
        g = torch.Generator().manual_seed(seed + layer)
        p = {}
        for name in PARAM_ORDER:
            shp = shapes[name]
            std = 1.0 / math.sqrt(shp[1]) if len(shp) == 2 else 0.02
            p[name] = torch.randn(*shp, generator=g) * std
        out.append(p)
    return out


def make_dit_input(batch, latent, dim, seed=7100):
    """x [B, L, dim] (smooth field + noise) and a cotangent g of the same shape, fp32 CPU."""
    T, H, W = latent
    L = T * H * W
    g = torch.Generator().manual_seed(seed)
    coarse = torch.randn(batch, dim, math.ceil(T / 4), math.ceil(H / 4), math.ceil(W / 4),
                         generator=g)
    fld = F.interpolate(coarse, size=(T, H, W), mode="trilinear", align_corners=False)
    fld = fld.reshape(batch, dim, L).transpose(1, 2)
    x = (fld + 0.5 * torch.randn(batch, L, dim, generator=g)).contiguous()
    cot = torch.randn(batch, L, dim, generator=g)
    return x, cot
