"""GPU parity of the token-granular query pool (vmoba_select_tokens, vmoba_token_attn_*)
against the fp64 oracle (oracle/tokens.py).

- Selection: the token mask must equal the oracle's except pairs whose normalised score
  lies within 1e-4 (relative) of the oracle's cutoff v*.  The kernel's masses carry the
  fp32 score rounding (about 1e-6 relative), which on a pool of L * N_b entries can move
  the cut by a few neighbouring entries; those lie within the window.  The union lists must
  be exactly the union of the GPU's own token mask, and the stats consistent with it.
- Attention: on the oracle's token mask and union lists (injected), O and LSE and the fp32
  gradients against the literal L x L oracle, within the bf16 tolerance.
- A token whose row of the mask is empty gets O = 0 and LSE = -inf and no gradient.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import tokens as otok
from synthetic import CONFIGS, LayerSpec, make_layer_inputs
from block_sparse_attention_layer_amd import (
    Problem, vmoba_partition_pool, vmoba_select_tokens, vmoba_token_attn_bwd,
    vmoba_token_attn_fwd)

from _parity import TOL, csr_to_device, masks_from_csc, masks_from_csr, max_err, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WINDOW = 1e-4

CASES = [
    ("tiny_bf16", "tiny", {}, LayerSpec(2, (2, 4, 4)), 64, 2),
    ("small3d_192", "l3d_55k", dict(T=8, H=12, W=16), LayerSpec(2, (4, 6, 8)), 128, 3),
    ("small3d_216", "cycle_76k", dict(T=6, H=18, W=16), LayerSpec(2, (3, 9, 8)), 128, 2),
    ("small2d_168", "l2d_32k", dict(T=7, H=18, W=12), LayerSpec(1, (7, 6, 4)), 128, 2),
    ("small1d_120", "l1d_32k", dict(T=6, H=10, W=12), LayerSpec(0, (1, 10, 12)), 128, 2),
    ("many_blocks_3d", "l3d_55k", dict(T=8, H=12, W=32), LayerSpec(2, (2, 2, 2)), 64, 2),
    # two batch entries (head groups g = b*Hh + h of both)
    ("batch2_3d", "l3d_55k", dict(T=4, H=12, W=16, batch=2), LayerSpec(2, (4, 6, 8)), 128, 2),
    # the block-count limit: 1024 blocks of 8 tokens, 32 mask words per token
    ("max_blocks_3d", "l3d_55k", dict(T=8, H=32, W=32), LayerSpec(2, (2, 2, 2)), 64, 1),
    # block sizes around one key tile (32 keys at d = 128, 64 at d = 64): from one tile up,
    # a tile's keys lie at two list positions at most and the kernels take two mask bits
    # a tile; below, one bit a key
    ("tile_exact_32", "l3d_55k", dict(T=4, H=8, W=8), LayerSpec(2, (2, 4, 4)), 128, 2),
    ("straddle_40", "l3d_55k", dict(T=2, H=10, W=16), LayerSpec(2, (1, 5, 8)), 128, 2),
    ("tile_exact_64_d64", "l3d_55k", dict(T=4, H=8, W=16), LayerSpec(2, (2, 4, 8)), 64, 2),
    ("under_tile_48_d64", "l3d_55k", dict(T=4, H=8, W=12), LayerSpec(2, (2, 4, 6)), 64, 2),
]
IDS = [c[0] for c in CASES]


def bits_to_bool(mask_i32, nb):
    m = mask_i32.cpu().numpy().view(np.uint32)
    G, L, W = m.shape
    j = np.arange(nb)
    return ((m[:, :, j >> 5] >> (j & 31).astype(np.uint32)) & 1).astype(bool)


def bool_to_bits(mb):
    G, L, nb = mb.shape
    W = (nb + 31) // 32
    out = np.zeros((G, L, W), dtype=np.uint32)
    for j in range(nb):
        out[:, :, j >> 5] |= mb[:, :, j].astype(np.uint32) << np.uint32(j & 31)
    return torch.from_numpy(out.view(np.int32))


def _setup(case, tau=0.25):
    name, cfgname, lat, spec, hd, heads = case
    cfg = dict(CONFIGS[cfgname])
    cfg.update(lat)
    batch = lat.get("batch", 1)
    over = dict(lat, heads=heads, head_dim=hd, batch=batch)
    inp = make_layer_inputs(cfgname, 0, backward=True, shape_override=over, dtype="bf16")
    p = Problem(batch, heads, hd, cfg["T"], cfg["H"], cfg["W"], spec.layer_idx,
                tuple(spec.block), torch.bfloat16, torch.float32)
    mem = oracle.block_members(p.T, p.H, p.W, p.block)
    blk = oracle.block_of_token(mem, p.L)
    print(f"[token case {name}] L={p.L} N_b={mem.shape[0]} tau={tau}", flush=True)
    q, k = to_np(inp["q"]), to_np(inp["k"])
    mask, shat, stats = otok.select_tokens_all_heads(q, oracle.block_means(k, mem), tau, blk)
    return p, inp, mem, blk, mask, shat, stats


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_token_selection_matches_oracle(case):
    p, inp, mem, blk, mask, shat, stats = _setup(case)
    nb = mem.shape[0]
    q, k = inp["q"].to(DEV), inp["k"].to(DEV)
    _, kp = vmoba_partition_pool(p, q, k)
    sel = vmoba_select_tokens(p, q, kp, 0.25)
    torch.cuda.synchronize()
    gm = bits_to_bool(sel.token_mask, nb)             # [G, L, nb], g = b*Hh + h
    G = p.groups
    om = mask.reshape(G, p.L, nb)
    osh = shat.reshape(G, p.L, nb)
    bad = exempt = 0
    for g in range(G):
        v = stats[g]["v"]
        diff = gm[g] != om[g]
        near = np.abs(osh[g] - v) <= WINDOW * v
        bad += int((diff & ~near).sum())
        exempt += int((diff & near).sum())
    print(f"  mismatches {bad}, exempt {exempt}", flush=True)
    assert bad == 0
    assert gm[:, np.arange(p.L), blk].all()           # every token keeps its own block
    # union lists of the GPU's own token mask, CSR and CSC alike
    union = otok.union_block_mask(gm[None], mem)[0]
    assert (masks_from_csr(sel.row_ptr, sel.col_idx, nb) == union).all()
    assert (masks_from_csc(sel.col_ptr, sel.row_idx, nb) == union).all()
    hs = sel.head_stats.cpu().numpy()
    for g in range(G):
        assert hs[g, 1] == gm[g].sum()
        assert abs(hs[g, 0] - stats[g]["k"]) <= max(2, exempt)
        assert abs(hs[g, 2] - stats[g]["mass"]) <= 1e-4
        assert abs(hs[g, 3] - stats[g]["v"]) <= 1e-4 * stats[g]["v"] + 1e-9


def _token_attention(case, mask, blk, mem, p, inp, tm_override=None):
    nb = mem.shape[0]
    tm = mask if tm_override is None else tm_override
    union = otok.union_block_mask(tm, mem)
    rp, ci, cp, ri = csr_to_device(union, DEV)
    bits = bool_to_bits(tm.reshape(-1, tm.shape[2], tm.shape[3])).to(DEV)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    o, lse = vmoba_token_attn_fwd(p, q, k, v, rp, ci, bits)
    dq, dk, dv = vmoba_token_attn_bwd(p, q, k, v, o, lse, do, rp, ci, cp, ri, bits)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_token_attention_matches_oracle(case):
    p, inp, mem, blk, mask, shat, stats = _setup(case)
    o, lse, dq, dk, dv = _token_attention(case, mask, blk, mem, p, inp)
    qn, kn, vn, don = (to_np(inp[x]) for x in ("q", "k", "v", "do"))
    ro, rl = otok.token_attention_fwd(qn, kn, vn, mask, blk)
    rg = otok.token_attention_bwd(qn, kn, vn, ro, rl, don, mask, blk)
    tol = TOL[torch.bfloat16]
    assert max_err(to_np(o), ro) <= tol
    assert max_err(to_np(lse), rl) <= tol
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), rg):
        assert max_err(to_np(got), want) <= tol, name


def test_token_attention_empty_row_and_partial_blocks():
    case = CASES[1]
    p, inp, mem, blk, mask, shat, stats = _setup(case)
    tm = mask.copy()
    x0 = 5
    tm[0, :, x0, :] = False                           # token 5 attends to nothing
    o, lse, dq, dk, dv = _token_attention(case, mask, blk, mem, p, inp, tm_override=tm)
    on, ln, dqn = to_np(o), to_np(lse), to_np(dq)
    assert (on[0, x0] == 0).all() and np.isneginf(ln[0, :, x0]).all() and (dqn[0, x0] == 0).all()
    keep = np.ones(p.L, bool)
    keep[x0] = False
    qn, kn, vn, don = (to_np(inp[x]) for x in ("q", "k", "v", "do"))
    tm2 = tm.copy()
    tm2[0, :, x0, :] = mask[0, :, x0, :]              # oracle rows need a key; row x0 unused
    ro, rl = otok.token_attention_fwd(qn, kn, vn, tm2, blk)
    ro[0, x0] = 0.0
    don0 = don.copy()
    don0[0, x0] = 0.0                                 # dO of the empty row plays no part
    rg = otok.token_attention_bwd(qn, kn, vn, ro, rl, don0, tm2, blk)
    tol = TOL[torch.bfloat16]
    assert max_err(on[:, keep], ro[:, keep]) <= tol
    assert max_err(ln[:, :, keep], rl[:, :, keep]) <= tol
    assert max_err(dqn[:, keep], rg[0][:, keep]) <= tol
    # dK/dV: the empty row contributes nothing; the GPU used the upstream dO of that row,
    # which with no selected pair must not reach dK/dV
    assert max_err(to_np(dk), rg[1]) <= tol
    assert max_err(to_np(dv), rg[2]) <= tol
