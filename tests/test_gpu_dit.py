"""The attention layer inside DiT blocks on the GPU against the oracle's fp64 block.

- One block per partition mode (1D, 2D, 3D) and per selection strategy, fp32: the
  block's own selection must equal the oracle's except pairs within 1e-5 of their pool's
  cutoff (then the oracle's lists are injected), and the output and the gradients of the
  input and of every weight must match.
- A bf16 stack of three layers (1D -> 2D -> 3D) through the warm-up switch: step 0 of 4
  runs the dense kernels in every layer, step 1 the block-sparse ones (on the oracle's
  selections, injected, since bf16 projections move scores near the cutoff).
Weights and inputs are the seeded draws of ``synthetic.dit``, cast to the compute dtype
before either side sees them.
"""

import numpy as np
import pytest
import torch

from oracle import dit as odit
from synthetic import make_dit_input, make_dit_params
from block_sparse_attention_layer_amd import LayerCycle, SyntheticDiT, SyntheticDiTBlock

from _parity import MASK_WINDOW, csr_to_device, masks_from_csc, masks_from_csr

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rel(a, b):
    """max |a - b| relative to max(1, max |b|)."""
    a = a.detach().double().cpu()
    b = b.detach().double().cpu()
    return float((a - b).abs().max()) / max(1.0, float(b.abs().max()))


def _mask_diffs(mode, gm, mask, shat, stats):
    B, Hh, nb, _ = mask.shape
    gm = gm.reshape(B, Hh, nb, nb)
    bad = exempt = 0
    for b in range(B):
        for h in range(Hh):
            st = stats[b * Hh + h]
            cut = (np.full((nb, 1), st["v"]) if mode.endswith("global")
                   else np.asarray(st["row_v"])[:, None])
            diff = gm[b, h] != mask[b, h]
            near = np.abs(shat[b, h] - cut) <= MASK_WINDOW
            bad += int((diff & ~near).sum())
            exempt += int((diff & near).sum())
    return bad, exempt


LAT = (4, 8, 8)
HEADS, HD = 2, 64
DIM, HID = HEADS * HD, 256
CYCLE = LayerCycle(LAT, (1, 8, 8), (4, 4, 4), (2, 4, 4))   # 4, 4 and 8 blocks of 64 / 32
STRATEGIES = [("threshold_global", 0.25, None), ("topk_global", None, 6),
              ("threshold_local", 0.3, None), ("topk_local", None, 2)]


@pytest.mark.parametrize("layer", [0, 1, 2], ids=["1d", "2d", "3d"])
@pytest.mark.parametrize("strategy", STRATEGIES, ids=[s[0] for s in STRATEGIES])
def test_block_fp32_matches_oracle(layer, strategy):
    mode, tau, k = strategy
    print(f"[dit block fp32 layer {layer} {mode}]", flush=True)
    P = make_dit_params(DIM, HID, 3)[layer]
    x, g = make_dit_input(1, LAT, DIM)
    blk = SyntheticDiTBlock(DIM, HEADS, HID, layer, CYCLE, tau=tau, mode=mode, topk=k,
                            dtype=torch.float32, device=DEV).load_params(P)
    # oracle, fp64 on the CPU, its own selection
    Po = {n: t.double().requires_grad_() for n, t in P.items()}
    xo = x.double().requires_grad_()
    yo, info = odit.dit_block(xo, Po, LAT, HEADS, layer, CYCLE.block(layer), tau=tau,
                              mode=mode, k_top=k)
    (yo * g.double()).sum().backward()
    # GPU block, its own selection
    xg = x.to(DEV).requires_grad_()
    y = blk(xg)
    torch.cuda.synchronize()
    assert blk.last_path == "sparse"
    nb = info["mask"].shape[-1]
    sel = blk.last_selection
    gm = masks_from_csr(sel.row_ptr, sel.col_idx, nb)
    assert (masks_from_csc(sel.col_ptr, sel.row_idx, nb) == gm).all()
    bad, exempt = _mask_diffs(mode, gm, info["mask"], info["shat"], info["stats"])
    assert bad == 0, f"{bad} selection mismatches"
    if exempt:   # near-ties at the cutoff: run on the oracle's lists
        blk.zero_grad()
        xg = x.to(DEV).requires_grad_()
        y = blk(xg, selection=csr_to_device(info["mask"], DEV))
    y.backward(g.to(DEV))
    torch.cuda.synchronize()
    tol = 2e-4
    assert _rel(y, yo) <= tol
    assert _rel(xg.grad, xo.grad) <= tol
    for mod, w, b in ((blk.q, "wq", "bq"), (blk.k, "wk", "bk"), (blk.v, "wv", "bv"),
                      (blk.o, "wo", "bo"), (blk.fc1, "w1", "b1"), (blk.fc2, "w2", "b2")):
        assert _rel(mod.weight.grad, Po[w].grad) <= tol, w
        assert _rel(mod.bias.grad, Po[b].grad) <= tol, b


LAT2 = (8, 8, 16)                       # 1,024 tokens
HEADS2, HD2 = 4, 128
DIM2, HID2 = HEADS2 * HD2, 1024
BLOCKS2 = [(2, 8, 16), (8, 4, 4), (2, 4, 8)]   # 4 / 8 / 16 blocks of 256 / 128 / 64
CYCLE2 = LayerCycle(LAT2, *BLOCKS2)


def _bf16_inputs():
    P = [{n: t.to(torch.bfloat16) for n, t in p.items()}
         for p in make_dit_params(DIM2, HID2, 3, seed=7200)]
    x, g = make_dit_input(1, LAT2, DIM2, seed=7300)
    return P, x.to(torch.bfloat16), g.to(torch.bfloat16)


@pytest.mark.parametrize("step", [0, 1], ids=["warmup_full", "sparse"])
def test_stack_bf16_cycle_and_warmup(step):
    print(f"[dit stack bf16 step {step} of 4]", flush=True)
    P, x, g = _bf16_inputs()
    Po = [{n: t.double().requires_grad_() for n, t in p.items()} for p in P]
    xo = x.double().requires_grad_()
    yo, infos = odit.dit_stack(xo, Po, LAT2, HEADS2, BLOCKS2, tau=0.25, step=step,
                               num_steps=4)
    (yo * g.double()).sum().backward()
    model = SyntheticDiT(3, DIM2, HEADS2, HID2, CYCLE2, tau=0.25, dtype=torch.bfloat16,
                         device=DEV).load_params(P)
    sels = None if step == 0 else [csr_to_device(inf["mask"], DEV) for inf in infos]
    xg = x.to(DEV).requires_grad_()
    y = model(xg, step=step, num_steps=4, selections=sels)
    y.backward(g.to(DEV))
    torch.cuda.synchronize()
    want = "dense" if step == 0 else "sparse"
    assert [b.last_path for b in model.blocks] == [want] * 3
    if step:
        assert [inf["members"].shape[0] for inf in infos] == [CYCLE2.num_blocks(l)
                                                              for l in range(3)]
    tol = 3e-2
    assert _rel(y, yo) <= tol
    assert _rel(xg.grad, xo.grad) <= tol
    for blk, po in zip(model.blocks, Po):
        for mod, w in ((blk.q, "wq"), (blk.k, "wk"), (blk.v, "wv"), (blk.o, "wo"),
                       (blk.fc1, "w1"), (blk.fc2, "w2")):
            assert _rel(mod.weight.grad, po[w].grad) <= tol, (blk.layer_idx, w)


def test_stack_bf16_own_selection_runs_the_layer_cycle():
    """Without injected lists each layer selects on its own partition: the lists have the
    layer's block count, keep every diagonal pair and are consistent between CSR and CSC."""
    P, x, g = _bf16_inputs()
    model = SyntheticDiT(3, DIM2, HEADS2, HID2, CYCLE2, tau=0.25, dtype=torch.bfloat16,
                         device=DEV).load_params(P)
    xg = x.to(DEV).requires_grad_()
    y = model(xg, step=3, num_steps=4)
    y.backward(g.to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(xg.grad).all()
    for layer, blk in enumerate(model.blocks):
        nb = CYCLE2.num_blocks(layer)
        s = blk.last_selection
        assert tuple(s.row_ptr.shape) == (HEADS2, nb + 1)
        gm = masks_from_csr(s.row_ptr, s.col_idx, nb)
        assert (masks_from_csc(s.col_ptr, s.row_idx, nb) == gm).all()
        assert gm[:, np.arange(nb), np.arange(nb)].all()


def test_block_fp32_batch2_matches_oracle():
    """Two batch entries: each is its own pool (head groups g = b*Hh + h)."""
    print("[dit block fp32 batch 2, 3D layer]", flush=True)
    layer = 2
    P = make_dit_params(DIM, HID, 3)[layer]
    x, g = make_dit_input(2, LAT, DIM, seed=7150)
    blk = SyntheticDiTBlock(DIM, HEADS, HID, layer, CYCLE, tau=0.25, dtype=torch.float32,
                            device=DEV).load_params(P)
    Po = {n: t.double().requires_grad_() for n, t in P.items()}
    xo = x.double().requires_grad_()
    yo, info = odit.dit_block(xo, Po, LAT, HEADS, layer, CYCLE.block(layer), tau=0.25)
    (yo * g.double()).sum().backward()
    xg = x.to(DEV).requires_grad_()
    y = blk(xg, selection=csr_to_device(info["mask"], DEV))
    y.backward(g.to(DEV))
    torch.cuda.synchronize()
    tol = 2e-4
    assert _rel(y, yo) <= tol
    assert _rel(xg.grad, xo.grad) <= tol
    for mod, w in ((blk.q, "wq"), (blk.k, "wk"), (blk.v, "wv"), (blk.o, "wo")):
        assert _rel(mod.weight.grad, Po[w].grad) <= tol, w
