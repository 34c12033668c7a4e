"""The attention layer inside a DiT block stack: the 1D -> 2D -> 3D layer cycle and the
full-attention warm-up.

papernotes 关键设计 1: layer l partitions the latent by l mod 3 (0: 1D, whole frames;
1: 2D, spatial patches across all frames; 2: 3D, spatio-temporal blocks), so one block
shape per mode serves every layer.  papernotes 损失函数/训练策略: the first 25 % of the
denoising steps keep full attention.  The projections and the MLP around the attention
are plain torch layers (the attention is the library's); their weights are supplied by
the caller (random ones stand in for a trained model).
"""

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import torch
import torch.nn.functional as F

from .api import Problem, vmoba_validate
from .layer import ListsLike, full_attention, vmoba_attention

MODES = ("1d", "2d", "3d")


@dataclass(frozen=True)
class LayerCycle:
    """Block shapes (b_t, b_h, b_w) for the 1D, 2D and 3D layers of a latent (T, H, W)."""
    latent: Tuple[int, int, int]
    block_1d: Tuple[int, int, int]
    block_2d: Tuple[int, int, int]
    block_3d: Tuple[int, int, int]

    def __post_init__(self):
        for layer, blk in enumerate((self.block_1d, self.block_2d, self.block_3d)):
            T, H, W = self.latent
            p = Problem(1, 1, 64, T, H, W, layer, tuple(blk))
            if vmoba_validate(p) != 0:
                raise ValueError(f"block {blk} is not a valid {MODES[layer]} partition of "
                                 f"latent {self.latent}")

    @staticmethod
    def mode(layer_idx: int) -> str:
        if layer_idx < 0:
            raise ValueError("layer index must be >= 0")
        return MODES[layer_idx % 3]

    def block(self, layer_idx: int) -> Tuple[int, int, int]:
        return (self.block_1d, self.block_2d, self.block_3d)[MODES.index(self.mode(layer_idx))]

    def num_blocks(self, layer_idx: int) -> int:
        T, H, W = self.latent
        bt, bh, bw = self.block(layer_idx)
        return (T // bt) * (H // bh) * (W // bw)


def full_attention_step(step: int, num_steps: int, warmup: float = 0.25) -> bool:
    """True for the denoising steps that keep full attention: the first ``warmup``
    fraction of the ``num_steps`` steps (step < warmup * num_steps; steps count from 0 in
    the order they are run, so 13 of 50 steps are full at 25 %)."""
    if not 0 <= step < num_steps:
        raise ValueError(f"step {step} outside [0, {num_steps})")
    if not 0.0 <= warmup <= 1.0:
        raise ValueError("warmup fraction must lie in [0, 1]")
    return step < warmup * num_steps


def num_full_steps(num_steps: int, warmup: float = 0.25) -> int:
    return sum(full_attention_step(s, num_steps, warmup) for s in range(num_steps))


class SyntheticDiTBlock(torch.nn.Module):
    """x + Attn(LN(x)) W_o, then + MLP(LN(.)): pre-norm self-attention and a GELU MLP.

    The attention takes q, k, v [B, L, Hh, d] straight from the [B, L, dim] projections
    (dim = Hh * d, head h = channels h*d .. h*d + d - 1), which is the layout the kernels
    use, so no copy sits between the projections and the attention.
    """

    def __init__(self, dim: int, heads: int, mlp_hidden: int, layer_idx: int,
                 cycle: LayerCycle, *, tau: float = 0.25, mode: str = "threshold_global",
                 topk: Optional[int] = None, dtype=torch.bfloat16, device="cuda"):
        super().__init__()
        if dim % heads:
            raise ValueError("dim must be a multiple of heads")
        self.dim, self.heads, self.head_dim = dim, heads, dim // heads
        self.layer_idx, self.cycle = layer_idx, cycle
        self.tau, self.mode, self.topk = tau, mode, topk
        kw = dict(dtype=dtype, device=device)
        lin = lambda i, o: torch.nn.Linear(i, o, bias=True, **kw)
        self.q, self.k, self.v, self.o = lin(dim, dim), lin(dim, dim), lin(dim, dim), lin(dim, dim)
        self.fc1, self.fc2 = lin(dim, mlp_hidden), lin(mlp_hidden, dim)
        self.last_path = None        # "sparse" or "dense": what the last forward ran
        self.last_selection = None   # lists of the last sparse forward

    def load_params(self, p: Dict[str, torch.Tensor]):
        """Copy weights given as {wq, bq, ..., w2, b2} (Linear layout [out, in])."""
        with torch.no_grad():
            for mod, w, b in ((self.q, "wq", "bq"), (self.k, "wk", "bk"), (self.v, "wv", "bv"),
                              (self.o, "wo", "bo"), (self.fc1, "w1", "b1"),
                              (self.fc2, "w2", "b2")):
                mod.weight.copy_(p[w])
                mod.bias.copy_(p[b])
        return self

    def forward(self, x, *, full: bool = False, selection: Optional[ListsLike] = None):
        B, L, _ = x.shape
        latent = self.cycle.latent
        h = F.layer_norm(x, (self.dim,), eps=1e-6)
        shp = (B, L, self.heads, self.head_dim)
        q, k, v = (m(h).view(shp) for m in (self.q, self.k, self.v))
        if full:
            a = full_attention(q, k, v, latent=latent)
            self.last_path, self.last_selection = "dense", None
        else:
            a, sel = vmoba_attention(q, k, v, latent=latent, layer_idx=self.layer_idx,
                                     block=self.cycle.block(self.layer_idx), tau=self.tau,
                                     mode=self.mode, topk=self.topk, selection=selection,
                                     return_selection=True)
            self.last_path, self.last_selection = "sparse", sel
        x = x + self.o(a.reshape(B, L, self.dim))
        h = F.layer_norm(x, (self.dim,), eps=1e-6)
        return x + self.fc2(F.gelu(self.fc1(h), approximate="tanh"))


class SyntheticDiT(torch.nn.Module):
    """A stack of blocks with layer indices 0 .. n-1, so the partitions cycle 1D, 2D, 3D,
    and the warm-up switch: full attention in every layer on the first steps."""

    def __init__(self, num_layers: int, dim: int, heads: int, mlp_hidden: int,
                 cycle: LayerCycle, *, warmup: float = 0.25, **block_kw):
        super().__init__()
        self.warmup = warmup
        self.blocks = torch.nn.ModuleList(
            SyntheticDiTBlock(dim, heads, mlp_hidden, layer, cycle, **block_kw)
            for layer in range(num_layers))

    def load_params(self, params: Sequence[Dict[str, torch.Tensor]]):
        if len(params) != len(self.blocks):
            raise ValueError("one parameter dict per block")
        for blk, p in zip(self.blocks, params):
            blk.load_params(p)
        return self

    def forward(self, x, *, step: Optional[int] = None, num_steps: Optional[int] = None,
                selections: Optional[List[Optional[ListsLike]]] = None):
        full = step is not None and full_attention_step(step, num_steps, self.warmup)
        for i, blk in enumerate(self.blocks):
            x = blk(x, full=full, selection=None if selections is None else selections[i])
        return x
