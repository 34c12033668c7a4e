"""Seeded generators (random draws only; no step of the method lives here)."""

import math

import torch
import torch.nn.functional as F

from .configs import CONFIGS, CONFIG_ORDER


def seed_for(config, layer_in_cycle=0):
    return 1000 * CONFIG_ORDER.index(config) + layer_in_cycle


_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


def make_layer_inputs(config, layer_in_cycle=0, *, backward=None, seed=None,
                      shape_override=None, dtype=None, field=None):
    """Q, K, V (and dO) for one layer of a workload, as CPU tensors [B, L, Hh, d].

    ``shape_override`` (dict with any of batch, heads, head_dim, T, H, W)
    reuses a workload's recipe at another size, for parity cases the oracle
    finishes in seconds.  Returns a dict q, k, v, do (None when no backward).
    """
    cfg = dict(CONFIGS[config])
    if shape_override:
        cfg.update(shape_override)
    B, Hh, d = cfg["batch"], cfg["heads"], cfg["head_dim"]
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    L = T * H * W
    want_bwd = cfg["backward"] if backward is None else backward
    field = field or cfg["field"]
    out_dtype = _DTYPES[dtype or cfg["dtype"]]
    g = torch.Generator().manual_seed(seed_for(config, layer_in_cycle)
                                      if seed is None else seed)
    if field == "iid":
        q = torch.randn(B, L, Hh, d, generator=g)
        k = torch.randn(B, L, Hh, d, generator=g)
    else:
        coarse = torch.randn(B, Hh * d, math.ceil(T / 4), math.ceil(H / 4),
                             math.ceil(W / 4), generator=g)
        fld = F.interpolate(coarse, size=(T, H, W), mode="trilinear",
                            align_corners=False)
        fld = fld.reshape(B, Hh, d, T, H, W).permute(0, 3, 4, 5, 1, 2)
        fld = fld.reshape(B, L, Hh, d)
        q = fld + 0.5 * torch.randn(B, L, Hh, d, generator=g)
        k = fld + 0.5 * torch.randn(B, L, Hh, d, generator=g)
        del fld, coarse
    v = torch.randn(B, L, Hh, d, generator=g)
    do = torch.randn(B, L, Hh, d, generator=g) if want_bwd else None
    cast = lambda t: None if t is None else t.to(out_dtype).contiguous()
    return {"q": cast(q), "k": cast(k), "v": cast(v), "do": cast(do)}
