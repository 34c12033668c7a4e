"""GPU parity of every stage against the fp64 oracle, at sizes the oracle finishes in
seconds that still span several tiles and ragged tails.

Attention is compared under the oracle's own block mask, passed to the kernels as a
row/column list, so selection differences cannot leak into attention errors; the
GPU's own selection is compared with the oracle's separately.
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import CONFIGS, LayerSpec, make_layer_inputs
from block_sparse_attention_layer_amd import (
    Problem, vmoba_attention, vmoba_dense_attn_bwd, vmoba_dense_attn_fwd,
    vmoba_partition_pool, vmoba_select, vmoba_sparse_attn_bwd, vmoba_sparse_attn_bwd_delta,
    vmoba_sparse_attn_bwd_dkdv, vmoba_sparse_attn_bwd_dq, vmoba_sparse_attn_fwd)

from _parity import (TOL, compare_masks, csr_to_device, gpu_pool_select, masks_from_csc,
                     masks_from_csr, max_err, problem_for, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (name, recipe config, latent override, layer spec, tau, dtype, head_dim, batch)
CASES = [
    ("tiny", "tiny", {}, LayerSpec(2, (2, 4, 4)), 0.25, "fp32", 64, 1),
    ("tiny_bf16", "tiny", {}, LayerSpec(2, (2, 4, 4)), 0.25, "bf16", 64, 1),
    ("small3d_192", "l3d_55k", dict(T=8, H=12, W=16), LayerSpec(2, (4, 6, 8)), 0.25, "bf16", 128, 1),
    ("small3d_216", "cycle_76k", dict(T=6, H=18, W=16), LayerSpec(2, (3, 9, 8)), 0.25, "bf16", 128, 1),
    # 256-token blocks: every wave of the eight-wave 32-query forward holds queries
    ("small3d_256", "l3d_55k", dict(T=8, H=16, W=16), LayerSpec(2, (4, 8, 8)), 0.4, "bf16", 128, 1),
    ("small2d_168", "l2d_32k", dict(T=7, H=18, W=12), LayerSpec(1, (7, 6, 4)), 0.25, "bf16", 128, 1),
    ("small1d_120", "l1d_32k", dict(T=6, H=10, W=12), LayerSpec(0, (1, 10, 12)), 0.25, "bf16", 128, 1),
    ("small3d_d64_b2", "l3d_55k", dict(T=8, H=12, W=16), LayerSpec(2, (4, 6, 8)), 0.5, "bf16", 64, 2),
    ("small3d_fp32", "l3d_55k", dict(T=4, H=12, W=16), LayerSpec(2, (2, 6, 8)), 0.3, "fp32", 128, 1),
    # d = 128, 192-token blocks, two batch entries: the split dK/dV and dQ kernels over
    # head groups of both
    ("small3d_192_b2", "l3d_55k", dict(T=8, H=12, W=16), LayerSpec(2, (4, 6, 8)), 0.8, "bf16", 128, 2),
    # 12 blocks of 384: two 192-row tiles per block in the 48-wide forward and dK/dV
    # kernels, three 128-query tiles in dQ (a launch this small keeps the 32-query dQ),
    # and a block count that is no multiple of 8
    ("tiles2_3d_384", "l3d_55k", dict(T=8, H=36, W=16), LayerSpec(2, (4, 12, 8)), 0.6, "bf16", 128, 1),
    # 576 blocks of 8: above the block count up to which launches rank the lists
    ("unranked_576_blocks", "l3d_55k", dict(T=8, H=18, W=32), LayerSpec(2, (2, 2, 2)), 0.97, "bf16", 128, 1),
]
IDS = [c[0] for c in CASES]


def _setup(case, heads=None):
    name, cfgname, lat, spec, tau, dt, hd, batch = case
    cfg = dict(CONFIGS[cfgname])
    cfg.update(lat)
    heads = heads or (2 if cfgname == "tiny" else 4)
    over = dict(lat, heads=heads, head_dim=hd, batch=batch)
    inp = make_layer_inputs(cfgname, 0, backward=True, shape_override=over, dtype=dt)
    dtype = torch.float32 if dt == "fp32" else torch.bfloat16
    # gradients come back as the fp32 accumulators: bf16 output rounding alone can
    # exceed the absolute tolerance once |dK| >= 8; the bf16 gradient mode is checked
    # against these bit for bit in test_bf16_gradients_are_rounded_fp32_gradients
    p = Problem(batch, heads, hd, cfg["T"], cfg["H"], cfg["W"], spec.layer_idx,
                tuple(spec.block), dtype, torch.float32)
    print(f"[case {name}] L={p.L} heads={heads} d={hd} block={spec.block} tau={tau}",
          flush=True)
    return p, inp, tau


@pytest.fixture(scope="module", params=CASES, ids=IDS)
def case(request):
    p, inp, tau = _setup(request.param)
    # oracle, from the same tensors upcast to fp64
    qn, kn, vn, dn = (to_np(inp[x]) for x in ("q", "k", "v", "do"))
    ref = oracle.oracle_layer(qn, kn, vn, p.T, p.H, p.W, p.layer_idx, p.block, tau, do=dn)
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}
    return p, tau, dev, ref


def test_pool_matches_block_means(case):
    p, tau, d, ref = case
    qp, kp = vmoba_partition_pool(p, d["q"], d["k"])
    torch.cuda.synchronize()
    tol = 2e-5 if p.dtype == torch.bfloat16 else 1e-5
    assert max_err(to_np(qp), ref["q_pool"]) <= tol
    assert max_err(to_np(kp), ref["k_pool"]) <= tol


def test_selection_matches_oracle(case):
    p, tau, d, ref = case
    qp, kp, sel = gpu_pool_select(p, d["q"], d["k"], tau, want_scores=True)
    nb = ref["mask"].shape[-1]
    gm = masks_from_csr(sel.row_ptr, sel.col_idx, nb)
    gmc = masks_from_csc(sel.col_ptr, sel.row_idx, nb)
    assert (gm == gmc).all(), "CSR and CSC disagree"
    bad, exempt = compare_masks(gm, ref["mask"], ref["shat"], ref["stats"])
    print(f"mask mismatches={bad} exempt={exempt}")
    assert bad == 0
    # normalised scores and per-head statistics
    G = p.groups
    shat = ref["shat"].reshape(G, nb, nb)
    # fp32 scores carry about sqrt(d) 2^-24 of sum |qbar_i kbar_i|, which exp(s - max)
    # turns into a relative error: 1e-6 absolute plus 3e-5 relative (the means of small
    # blocks have the largest scores)
    ns = to_np(sel.norm_scores)
    ratio = float(np.max(np.abs(ns - shat) / (1e-6 + 3e-5 * np.abs(shat))))
    print(f"normalised scores: max-abs {max_err(ns, shat):.3g}, max ratio to bound {ratio:.3g}")
    assert ratio <= 1.0
    hs = sel.head_stats.cpu().numpy()
    for g in range(G):
        st = ref["stats"][g]
        assert hs[g, 1] == gm[g].sum()
        if exempt == 0:
            assert int(hs[g, 0]) == st["k"]
            assert hs[g, 2] == pytest.approx(st["mass"], abs=1e-5)
            assert hs[g, 3] == pytest.approx(st["v"], abs=1e-6)
        assert hs[g, 2] >= tau - 1e-6
    # columns ascending, diagonal present
    rp = sel.row_ptr.cpu().numpy()
    ci = sel.col_idx.cpu().numpy()
    for g in range(G):
        for i in range(nb):
            cols = ci[g, rp[g, i]:rp[g, i + 1]]
            assert (np.diff(cols) > 0).all() and i in cols


def test_forward_under_oracle_mask(case):
    p, tau, d, ref = case
    rp, ci, cp, ri = csr_to_device(ref["mask"], DEV)
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], rp, ci)
    torch.cuda.synchronize()
    tol = TOL[p.dtype]
    eo = max_err(to_np(o), ref["o"])
    el = max_err(to_np(lse), ref["lse"])
    print(f"fwd max-abs O={eo:.3g} LSE={el:.3g}")
    assert eo <= tol and el <= tol


def test_backward_under_oracle_mask(case):
    p, tau, d, ref = case
    rp, ci, cp, ri = csr_to_device(ref["mask"], DEV)
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], rp, ci)
    dq, dk, dv = vmoba_sparse_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"], rp, ci,
                                       cp, ri)
    torch.cuda.synchronize()
    tol = TOL[p.dtype]
    errs = {n: max_err(to_np(t), ref[n]) for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    print("bwd max-abs", {k: f"{v:.3g}" for k, v in errs.items()})
    for n, e in errs.items():
        assert e <= tol, (n, e)


def test_bwd_stage_calls_equal_combined_call(case):
    p, tau, d, ref = case
    rp, ci, cp, ri = csr_to_device(ref["mask"], DEV)
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], rp, ci)
    g = vmoba_sparse_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"], rp, ci, cp, ri)
    delta = vmoba_sparse_attn_bwd_delta(p, o, d["do"])
    dq = vmoba_sparse_attn_bwd_dq(p, d["q"], d["k"], d["v"], lse, delta, d["do"], rp, ci)
    dk, dv = vmoba_sparse_attn_bwd_dkdv(p, d["q"], d["k"], d["v"], lse, delta, d["do"], cp, ri)
    torch.cuda.synchronize()
    # delta against its definition on the returned O
    ref_delta = (o.double() * d["do"].double()).sum(-1).permute(0, 2, 1)
    assert float((delta.double() - ref_delta).abs().max()) <= 1e-3
    for a, b in zip(g, (dq, dk, dv)):
        assert torch.equal(a, b)


def test_deterministic(case):
    p, tau, d, ref = case
    outs = []
    for _ in range(2):
        qp, kp, sel = gpu_pool_select(p, d["q"], d["k"], tau)
        o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], sel.row_ptr, sel.col_idx)
        g = vmoba_sparse_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"], sel.row_ptr,
                                  sel.col_idx, sel.col_ptr, sel.row_idx)
        torch.cuda.synchronize()
        nb = sel.row_ptr.shape[1] - 1
        lists = [masks_from_csr(sel.row_ptr, sel.col_idx, nb),
                 masks_from_csc(sel.col_ptr, sel.row_idx, nb)]
        outs.append([qp, kp, sel.row_ptr, sel.col_ptr, sel.head_stats, o, lse, *g, lists])
    for a, b in zip(outs[0][:-1], outs[1][:-1]):
        assert torch.equal(a, b)
    for a, b in zip(outs[0][-1], outs[1][-1]):
        assert (a == b).all()


def test_bf16_gradients_are_rounded_fp32_gradients(case):
    p, tau, d, ref = case
    if p.dtype != torch.bfloat16:
        pytest.skip("fp32 inputs return fp32 gradients")
    rp, ci, cp, ri = csr_to_device(ref["mask"], DEV)
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], rp, ci)
    g32 = vmoba_sparse_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"], rp, ci, cp, ri)
    p16 = Problem(p.batch, p.heads, p.head_dim, p.T, p.H, p.W, p.layer_idx, p.block,
                  torch.bfloat16, torch.bfloat16)
    g16 = vmoba_sparse_attn_bwd(p16, d["q"], d["k"], d["v"], o, lse, d["do"], rp, ci, cp, ri)
    torch.cuda.synchronize()
    for a, b in zip(g32, g16):
        assert b.dtype == torch.bfloat16
        assert torch.equal(a.to(torch.bfloat16), b)   # torch's cast rounds to nearest even


def test_layer_autograd_end_to_end(case):
    p, tau, d, ref = case
    q, k, v = (d[x].clone().requires_grad_() for x in ("q", "k", "v"))
    o = vmoba_attention(q, k, v, latent=(p.T, p.H, p.W), layer_idx=p.layer_idx,
                        block=p.block, tau=tau)
    o.backward(d["do"])
    torch.cuda.synchronize()
    # the autograd path is the C ABI sequence with the layer's own selection; its
    # gradients (in the input dtype) are the rounded fp32 gradients of that sequence
    qp, kp, sel = gpu_pool_select(p, d["q"], d["k"], tau)
    o2, lse2 = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], sel.row_ptr, sel.col_idx)
    g32 = vmoba_sparse_attn_bwd(p, d["q"], d["k"], d["v"], o2, lse2, d["do"], sel.row_ptr,
                                sel.col_idx, sel.col_ptr, sel.row_idx)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for t, r in zip((q.grad, k.grad, v.grad), g32):
        assert torch.equal(t, r.to(p.dtype))
    # and, where the selection equals the oracle's, the output matches the oracle
    nb = ref["mask"].shape[-1]
    gm = masks_from_csr(sel.row_ptr, sel.col_idx, nb).reshape(ref["mask"].shape)
    if (gm == ref["mask"]).all():
        assert max_err(to_np(o), ref["o"]) <= TOL[p.dtype]
        for n, t in (("dq", g32[0]), ("dk", g32[1]), ("dv", g32[2])):
            assert max_err(to_np(t), ref[n]) <= TOL[p.dtype], n


# ---------------------------------------------------------------------------------
# degenerate and edge cases

def _small(dtype=torch.bfloat16, hd=128, heads=2, lat=(4, 12, 16), block=(2, 6, 8), layer=2):
    inp = make_layer_inputs("l3d_55k", 0, backward=True,
                            shape_override=dict(T=lat[0], H=lat[1], W=lat[2], heads=heads,
                                                head_dim=hd),
                            dtype="fp32" if dtype == torch.float32 else "bf16")
    p = Problem(1, heads, hd, *lat, layer, block, dtype, torch.float32)
    return p, inp


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_tau_one_selects_all_and_equals_dense(dtype):
    p, inp = _small(dtype)
    d = {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}
    qp, kp, sel = gpu_pool_select(p, d["q"], d["k"], 1.0)
    nb = (p.T // p.block[0]) * (p.H // p.block[1]) * (p.W // p.block[2])
    assert masks_from_csr(sel.row_ptr, sel.col_idx, nb).all()
    o_s, l_s = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], sel.row_ptr, sel.col_idx)
    o_d, l_d = vmoba_dense_attn_fwd(p, d["q"], d["k"], d["v"])
    g_s = vmoba_sparse_attn_bwd(p, d["q"], d["k"], d["v"], o_s, l_s, d["do"], sel.row_ptr,
                                sel.col_idx, sel.col_ptr, sel.row_idx)
    g_d = vmoba_dense_attn_bwd(p, d["q"], d["k"], d["v"], o_d, l_d, d["do"])
    torch.cuda.synchronize()
    qn, kn, vn, dn = (to_np(inp[x]) for x in ("q", "k", "v", "do"))
    mem = oracle.block_members(p.T, p.H, p.W, p.block)
    full = np.ones((1, p.heads, nb, nb), dtype=bool)
    o_ref, lse_ref = oracle.sparse_attention_fwd(qn, kn, vn, mem, full)
    grads_ref = oracle.sparse_attention_bwd(qn, kn, vn, o_ref, lse_ref, dn, mem, full)
    tol = TOL[dtype]
    for o in (o_s, o_d):
        assert max_err(to_np(o), o_ref) <= tol
    for l in (l_s, l_d):
        assert max_err(to_np(l), lse_ref) <= tol
    for g in (g_s, g_d):
        for t, r in zip(g, grads_ref):
            assert max_err(to_np(t), r) <= tol


# lengths that are no multiple of any tile: 330 takes the 48-query forward and the split
# dK/dV and dQ kernels, 250 the 32-query ones
@pytest.mark.parametrize("lat", [(3, 10, 11), (2, 5, 25)], ids=["L330", "L250"])
def test_dense_natural_order_ragged_length(lat):
    p, inp = _small(lat=lat, block=lat, layer=2)
    d = {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}
    o, lse = vmoba_dense_attn_fwd(p, d["q"], d["k"], d["v"])
    dq, dk, dv = vmoba_dense_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"])
    torch.cuda.synchronize()
    qn, kn, vn, dn = (to_np(inp[x]) for x in ("q", "k", "v", "do"))
    tm = np.ones((1, p.heads, p.L, p.L), dtype=bool)
    o_ref, lse_ref = oracle.dense_masked_attention_fwd(qn, kn, vn, tm)
    g_ref = oracle.dense_masked_attention_bwd(qn, kn, vn, o_ref, lse_ref, dn, tm)
    assert max_err(to_np(o), o_ref) <= 2e-2
    assert max_err(to_np(lse), lse_ref) <= 2e-2
    for t, r in zip((dq, dk, dv), g_ref):
        assert max_err(to_np(t), r) <= 2e-2


def test_caller_lists_with_empty_row_and_bad_entries():
    p, inp = _small(heads=2)
    d = {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}
    nb = 2 * 2 * 2
    rng = np.random.default_rng(0)
    mask = rng.random((1, 2, nb, nb)) < 0.4
    mask[0, :, np.arange(nb), np.arange(nb)] = True
    mask[0, 1, 3, :] = False          # an empty query row
    rp, ci, cp, ri = (t.cpu() for t in csr_to_device(mask, "cpu"))
    # append an out-of-range column to row 0 of head 0 by shifting later entries
    rp2, ci2 = rp.clone(), ci.clone()
    end0 = int(rp[0, 1])
    ci2[0, end0 + 1:] = ci[0, end0:-1]
    ci2[0, end0] = nb + 5
    rp2[0, 1:] += 1
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], rp2.to(DEV), ci2.to(DEV))
    torch.cuda.synchronize()
    qn, kn, vn = (to_np(inp[x]) for x in ("q", "k", "v"))
    mem = oracle.block_members(p.T, p.H, p.W, p.block)
    empty_tok = mem[3]
    m2 = mask.copy()
    m2[0, 1, 3, 3] = True             # give the oracle a defined row there
    o_ref, lse_ref = oracle.sparse_attention_fwd(qn, kn, vn, mem, m2)
    on, ln = to_np(o), to_np(lse)
    keep = np.ones(p.L, dtype=bool)
    keep[empty_tok] = False
    assert max_err(on[:, :, 0], o_ref[:, :, 0]) <= 2e-2
    assert max_err(on[:, keep, 1], o_ref[:, keep, 1]) <= 2e-2
    assert np.all(on[0, empty_tok, 1] == 0.0)
    assert np.all(np.isneginf(ln[0, 1, empty_tok]))


def _append_bad_entry(ptr, idx, g, row, bad):
    """A copy of one head group's CSR (or CSC) with an out-of-range entry appended to one
    row (entries after it shift by one)."""
    ptr2, idx2 = ptr.clone(), idx.clone()
    end = int(ptr[g, row + 1])
    idx2[g, end + 1:] = idx[g, end:-1]
    idx2[g, end] = bad
    ptr2[g, row + 1:] += 1
    return ptr2, idx2


# 96-token blocks take the 32-wide kernels, 192-token blocks the 48-wide forward and the
# split dK/dV and dQ kernels
@pytest.mark.parametrize("lat,block", [((4, 12, 16), (2, 6, 8)), ((8, 12, 16), (4, 6, 8))],
                         ids=["S96", "S192"])
def test_caller_lists_backward_with_empty_row_and_bad_entries(lat, block):
    p, inp = _small(heads=2, lat=lat, block=block)
    nb = (lat[0] // block[0]) * (lat[1] // block[1]) * (lat[2] // block[2])
    mem = oracle.block_members(p.T, p.H, p.W, p.block)
    empty_tok = mem[3]
    # the empty row's queries get no upstream gradient: they then add nothing to dK and dV
    # and have dQ = 0, as the oracle's gradients with that row given its diagonal do too
    inp = dict(inp)
    do = inp["do"].clone()
    do[0, torch.as_tensor(empty_tok, dtype=torch.long), 1] = 0
    inp["do"] = do
    d = {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}
    rng = np.random.default_rng(1)
    mask = rng.random((1, 2, nb, nb)) < 0.4
    mask[0, :, np.arange(nb), np.arange(nb)] = True
    mask[0, 1, 3, :] = False          # an empty query row
    rp, ci, cp, ri = (t.cpu() for t in csr_to_device(mask, "cpu"))
    rp2, ci2 = _append_bad_entry(rp, ci, 0, 0, nb + 5)
    cp2, ri2 = _append_bad_entry(cp, ri, 0, 1, -7)
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], rp2.to(DEV), ci2.to(DEV))
    dq, dk, dv = vmoba_sparse_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"],
                                       rp2.to(DEV), ci2.to(DEV), cp2.to(DEV), ri2.to(DEV))
    torch.cuda.synchronize()
    qn, kn, vn, dn = (to_np(inp[x]) for x in ("q", "k", "v", "do"))
    m2 = mask.copy()
    m2[0, 1, 3, 3] = True
    o_ref, lse_ref = oracle.sparse_attention_fwd(qn, kn, vn, mem, m2)
    g_ref = oracle.sparse_attention_bwd(qn, kn, vn, o_ref, lse_ref, dn, mem, m2)
    for name, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        e = max_err(to_np(t), r)
        print(f"{name} max-abs {e:.3g}")
        assert e <= 2e-2, name
    assert np.all(to_np(dq)[0, empty_tok, 1] == 0.0)


def test_maximum_block_count_selection():
    # 1024 one-token blocks: the largest pool the selection accepts (1,048,576 pairs)
    p, inp = _small(heads=1, lat=(1, 32, 32), block=(1, 1, 1), layer=2)
    d = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    qp, kp, sel = gpu_pool_select(p, d["q"], d["k"], 0.25, want_scores=True)
    qn, kn = to_np(inp["q"]), to_np(inp["k"])
    mem = oracle.block_members(p.T, p.H, p.W, p.block)
    mask, shat, stats = oracle.select_all_heads(oracle.block_means(qn, mem),
                                                oracle.block_means(kn, mem), 0.25)
    gm = masks_from_csr(sel.row_ptr, sel.col_idx, 1024)
    bad, exempt = compare_masks(gm, mask, shat, stats)
    assert bad == 0
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], *csr_to_device(mask, DEV)[:2])
    torch.cuda.synchronize()
    o_ref, _ = oracle.sparse_attention_fwd(qn, kn, to_np(inp["v"]), mem, mask)
    assert max_err(to_np(o), o_ref) <= 2e-2
