"""GPU parity of the other selection strategies (top-k + global, threshold + local,
top-k + local; paperlayer §4.4, Table 3) against the fp64 oracle.

Masks must be identical except pairs whose normalised score lies within 1e-5 of the
cutoff of their pool: the head's pool for top-k + global, the row's pool for the local
strategies.  The attention kernels then run on the GPU's own lists and are compared with
the oracle's attention under the same mask.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synthetic import CONFIGS, LayerSpec, make_layer_inputs
from block_sparse_attention_layer_amd import (
    Problem, vmoba_partition_pool, vmoba_select, vmoba_sparse_attn_bwd, vmoba_sparse_attn_fwd)

from _parity import MASK_WINDOW, TOL, masks_from_csc, masks_from_csr, max_err, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    ("tiny_bf16", "tiny", {}, LayerSpec(2, (2, 4, 4)), 64),
    ("small3d_192", "l3d_55k", dict(T=8, H=12, W=16), LayerSpec(2, (4, 6, 8)), 128),
    ("small3d_216", "cycle_76k", dict(T=6, H=18, W=16), LayerSpec(2, (3, 9, 8)), 128),
    ("small2d_168", "l2d_32k", dict(T=7, H=18, W=12), LayerSpec(1, (7, 6, 4)), 128),
    ("many_blocks_3d", "l3d_55k", dict(T=8, H=12, W=32), LayerSpec(2, (2, 2, 2)), 64),
]
MODES = ["topk_global", "threshold_local", "topk_local"]


def _params(mode, nb):
    """tau / k giving roughly a fifth of the pairs."""
    if mode == "topk_global":
        return None, max(1, math.ceil(0.2 * nb * nb))
    if mode == "topk_local":
        return None, max(1, round(0.2 * nb))
    return 0.25, None


def _run(case, mode):
    name, cfgname, lat, spec, hd = case
    cfg = dict(CONFIGS[cfgname])
    cfg.update(lat)
    heads = 3
    over = dict(lat, heads=heads, head_dim=hd, batch=1)
    inp = make_layer_inputs(cfgname, 0, backward=True, shape_override=over, dtype="bf16")
    p = Problem(1, heads, hd, cfg["T"], cfg["H"], cfg["W"], spec.layer_idx, tuple(spec.block),
                torch.bfloat16, torch.float32)
    mem = oracle.block_members(p.T, p.H, p.W, p.block)
    nb = mem.shape[0]
    tau, k = _params(mode, nb)
    print(f"[case {name} mode {mode}] L={p.L} N_b={nb} tau={tau} k={k}", flush=True)
    q, kk = inp["q"].to(DEV), inp["k"].to(DEV)
    qp, kp = vmoba_partition_pool(p, q, kk)
    sel = vmoba_select(p, qp, kp, tau, want_scores=True, mode=mode, k=k)
    torch.cuda.synchronize()
    qn, kn = to_np(inp["q"]), to_np(inp["k"])
    mask, shat, stats = oracle.select_all_heads(oracle.block_means(qn, mem),
                                                oracle.block_means(kn, mem), tau, mode=mode, k=k)
    return p, inp, sel, mask, shat, stats, nb, tau, k


def _compare(mode, gm, mask, shat, stats):
    """(mismatches outside the cutoff window, mismatches inside it)."""
    B, Hh, nb, _ = mask.shape
    gm = gm.reshape(B, Hh, nb, nb)
    bad = exempt = 0
    for b in range(B):
        for h in range(Hh):
            st = stats[b * Hh + h]
            cut = (np.full((nb, 1), st["v"]) if mode == "topk_global"
                   else np.asarray(st["row_v"])[:, None])
            diff = gm[b, h] != mask[b, h]
            near = np.abs(shat[b, h] - cut) <= MASK_WINDOW
            bad += int((diff & ~near).sum())
            exempt += int((diff & near).sum())
    return bad, exempt


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_selection_mode_matches_oracle(case, mode):
    p, inp, sel, mask, shat, stats, nb, tau, k = _run(case, mode)
    gm = masks_from_csr(sel.row_ptr, sel.col_idx, nb)
    assert (gm == masks_from_csc(sel.col_ptr, sel.row_idx, nb)).all(), "CSR and CSC disagree"
    bad, exempt = _compare(mode, gm, mask, shat, stats)
    print(f"mask mismatches={bad} exempt={exempt}")
    assert bad == 0
    G = p.groups
    assert max_err(to_np(sel.norm_scores), shat.reshape(G, nb, nb)) <= 1e-6
    hs = sel.head_stats.cpu().numpy()
    rp = sel.row_ptr.cpu().numpy()
    ci = sel.col_idx.cpu().numpy()
    for g in range(G):
        st = stats[g]
        assert hs[g, 1] == gm[g].sum()
        if exempt == 0:
            assert int(hs[g, 0]) == st["k"]
            if mode == "topk_global":
                assert hs[g, 2] == pytest.approx(st["mass"], abs=1e-5)
                assert hs[g, 3] == pytest.approx(st["v"], abs=1e-6)
            else:
                assert hs[g, 2] == pytest.approx(np.mean(st["row_mass"]), abs=1e-5)
                assert hs[g, 3] == pytest.approx(np.mean(st["row_v"]), abs=1e-5)
        for i in range(nb):
            cols = ci[g, rp[g, i]:rp[g, i + 1]]
            assert (np.diff(cols) > 0).all() and i in cols
            if mode == "topk_local":   # exactly k, plus the diagonal when it is not among them
                assert len(cols) in (min(k, nb), min(k, nb) + 1)
    if mode == "topk_global":
        assert all(int(hs[g, 0]) == min(k, nb * nb) for g in range(G))


@pytest.mark.parametrize("mode", MODES)
def test_attention_on_mode_lists(mode):
    case = CASES[1]
    p, inp, sel, mask, shat, stats, nb, tau, k = _run(case, mode)
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}
    o, lse = vmoba_sparse_attn_fwd(p, dev["q"], dev["k"], dev["v"], sel.row_ptr, sel.col_idx)
    dq, dk, dv = vmoba_sparse_attn_bwd(p, dev["q"], dev["k"], dev["v"], o, lse, dev["do"],
                                       sel.row_ptr, sel.col_idx, sel.col_ptr, sel.row_idx)
    torch.cuda.synchronize()
    gm = masks_from_csr(sel.row_ptr, sel.col_idx, nb).reshape(1, p.heads, nb, nb)
    qn, kn, vn, dn = (to_np(inp[x]) for x in ("q", "k", "v", "do"))
    mem = oracle.block_members(p.T, p.H, p.W, p.block)
    ro, rlse = oracle.sparse_attention_fwd(qn, kn, vn, mem, gm)
    rdq, rdk, rdv = oracle.sparse_attention_bwd(qn, kn, vn, ro, rlse, dn, mem, gm)
    for name, got, ref in (("O", o, ro), ("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        e = max_err(to_np(got), ref)
        print(f"{mode} {name} max err {e:.3g}")
        assert e <= TOL[torch.bfloat16], name
