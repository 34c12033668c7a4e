"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark
times.

* pooling: every block mean against the oracle;
* selection: the whole mask against the oracle's (cutoff window exempt);
* attention under the oracle's mask: sampled query rows (O, LSE, dQ) and whole
  sampled key blocks (dK, dV) computed one by one from the definition, plus two
  identities that hold at any size: sum_y dV_y = sum_x dO_x (rows of P sum to one)
  and sum_y dK_y = 0 (rows of dS sum to zero when delta = rowsum(dO * O)).
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import CONFIGS, config_layers, make_layer_inputs
from block_sparse_attention_layer_amd import (Problem, vmoba_sparse_attn_bwd,
                                              vmoba_sparse_attn_fwd)

from _parity import (compare_masks, csr_to_device, gpu_pool_select, masks_from_csr,
                     max_err, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2

LAYERS = [(name, li) for name in ("l1d_32k", "l2d_32k", "l3d_55k", "cycle_76k", "blocks_55k",
                                  "blocks_46k", "blocks_11k")
          for li, _ in config_layers(name)]


@pytest.fixture(scope="module", params=LAYERS, ids=[f"{n}-L{li}" for n, li in LAYERS])
def layer(request):
    name, li = request.param
    cfg = CONFIGS[name]
    spec = cfg["layers"][li]
    print(f"[full-size {name} layer {li}] generating inputs", flush=True)
    inp = make_layer_inputs(name, li, backward=True)
    p = Problem(cfg["batch"], cfg["heads"], cfg["head_dim"], cfg["T"], cfg["H"], cfg["W"],
                spec.layer_idx, tuple(spec.block), torch.bfloat16, torch.float32)
    mem = oracle.block_members(p.T, p.H, p.W, p.block)
    qn, kn = to_np(inp["q"]), to_np(inp["k"])
    qpool, kpool = oracle.block_means(qn, mem), oracle.block_means(kn, mem)
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}
    return dict(name=name, cfg=cfg, p=p, inp=inp, dev=dev, mem=mem, qpool=qpool,
                kpool=kpool, blk=oracle.block_of_token(mem, p.L))


def test_pool_and_selection_full_size(layer):
    p, d = layer["p"], layer["dev"]
    for tau in layer["cfg"]["taus"]:
        print(f"tau={tau}", flush=True)
        qp, kp, sel = gpu_pool_select(p, d["q"], d["k"], tau)
        assert max_err(to_np(qp), layer["qpool"]) <= 2e-5
        assert max_err(to_np(kp), layer["kpool"]) <= 2e-5
        mask, shat, stats = oracle.select_all_heads(layer["qpool"], layer["kpool"], tau)
        nb = mask.shape[-1]
        gm = masks_from_csr(sel.row_ptr, sel.col_idx, nb)
        bad, exempt = compare_masks(gm, mask, shat, stats)
        density = gm.mean()
        print(f"  nnz density={density:.4f} mismatches={bad} exempt={exempt}")
        assert bad == 0


def test_attention_full_size_sampled(layer):
    p, d, mem, blk = layer["p"], layer["dev"], layer["mem"], layer["blk"]
    inp = layer["inp"]
    tau = 0.25
    mask, shat, stats = oracle.select_all_heads(layer["qpool"], layer["kpool"], tau)
    rp, ci, cp, ri = csr_to_device(mask, DEV)
    o, lse = vmoba_sparse_attn_fwd(p, d["q"], d["k"], d["v"], rp, ci)
    dq, dk, dv = vmoba_sparse_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"], rp, ci,
                                       cp, ri)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    q, k, v, do = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    on, ln, dqn = o.float().cpu().numpy(), lse.cpu().numpy(), dq.cpu().numpy()
    for h in (0, p.heads - 1):
        rows = np.sort(rng.choice(p.L, 48, replace=False))
        r = oracle.sampled_query_rows(q, k, v, do, mem, blk, mask, 0, h, rows)
        eo = max_err(on[0, rows, h], r["o"])
        el = max_err(ln[0, h, rows], r["lse"])
        eq = max_err(dqn[0, rows, h], r["dq"])
        print(f"head {h}: O {eo:.3g} LSE {el:.3g} dQ {eq:.3g}", flush=True)
        assert eo <= TOL and el <= TOL and eq <= TOL
    # whole key blocks: the median and the most-selected column of head 0
    colcnt = mask[0, 0].sum(axis=0)
    dkn, dvn = dk.cpu().numpy(), dv.cpu().numpy()
    for j in {int(np.argsort(colcnt)[len(colcnt) // 2]), int(np.argmax(colcnt))}:
        gk, gv = oracle.sampled_key_block_grads(q, k, v, do, mem, mask, 0, 0, j)
        ek = max_err(dkn[0, mem[j], 0], gk)
        ev = max_err(dvn[0, mem[j], 0], gv)
        print(f"key block {j} ({colcnt[j]} query blocks): dK {ek:.3g} dV {ev:.3g}",
              flush=True)
        assert ek <= TOL and ev <= TOL
    # identities over all keys of every head
    sum_dv = dv.double().sum(dim=1)
    sum_do = inp["do"].double().sum(dim=1).to(DEV)
    sum_dk = dk.double().sum(dim=1)
    e1 = float((sum_dv - sum_do).abs().max())
    e2 = float(sum_dk.abs().max())
    print(f"sum rules: |sum dV - sum dO| {e1:.3g}  |sum dK| {e2:.3g}")
    assert e1 <= 0.5 and e2 <= 0.5
    # the bf16 gradient mode the benchmark times returns these gradients rounded
    p16 = Problem(p.batch, p.heads, p.head_dim, p.T, p.H, p.W, p.layer_idx, p.block,
                  torch.bfloat16, torch.bfloat16)
    g16 = vmoba_sparse_attn_bwd(p16, d["q"], d["k"], d["v"], o, lse, d["do"], rp, ci, cp, ri)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), g16):
        assert torch.equal(a.to(torch.bfloat16), b)


def test_selection_modes_full_size(layer):
    """The ablation's other strategies (top-k + global, threshold + local, top-k + local)
    at full size: whole masks against the oracle, cutoff window exempt."""
    from block_sparse_attention_layer_amd import vmoba_partition_pool, vmoba_select
    from test_gpu_select_modes import _compare, _params
    p, d = layer["p"], layer["dev"]
    qp, kp = vmoba_partition_pool(p, d["q"], d["k"])
    nb = layer["mem"].shape[0]
    for mode in ("topk_global", "threshold_local", "topk_local"):
        tau, k = _params(mode, nb)
        sel = vmoba_select(p, qp, kp, tau, mode=mode, k=k)
        torch.cuda.synchronize()
        mask, shat, stats = oracle.select_all_heads(layer["qpool"], layer["kpool"], tau,
                                                    mode=mode, k=k)
        gm = masks_from_csr(sel.row_ptr, sel.col_idx, nb)
        bad, exempt = _compare(mode, gm, mask, shat, stats)
        print(f"  {mode} tau={tau} k={k} density={gm.mean():.4f} mismatches={bad} "
              f"exempt={exempt}", flush=True)
        assert bad == 0


@pytest.mark.parametrize("name,li", [("l3d_55k", 0), ("blocks_55k", 2)],
                         ids=["l3d_55k-L0", "blocks_55k-L2"])
def test_token_granular_full_size(name, li):
    """Token-granular pool at full length on two heads (heads are independent problems):
    the token mask against the oracle's (cutoff window 1e-4 relative), then the attention
    on the oracle's mask: sampled rows (O, LSE, dQ) and the two sum identities."""
    from oracle import tokens as otok
    from block_sparse_attention_layer_amd import (vmoba_partition_pool, vmoba_select_tokens,
                                                  vmoba_token_attn_bwd, vmoba_token_attn_fwd)
    from test_gpu_tokens import bits_to_bool, bool_to_bits
    cfg = CONFIGS[name]
    spec = cfg["layers"][li]
    print(f"[full-size token pool {name} layer {li}] generating inputs", flush=True)
    full = make_layer_inputs(name, li, backward=True)
    heads = [0, cfg["heads"] - 1]
    inp = {x: full[x][:, :, heads].contiguous() for x in ("q", "k", "v", "do")}
    del full
    p = Problem(cfg["batch"], len(heads), cfg["head_dim"], cfg["T"], cfg["H"], cfg["W"],
                spec.layer_idx, tuple(spec.block), torch.bfloat16, torch.float32)
    mem = oracle.block_members(p.T, p.H, p.W, p.block)
    blk = oracle.block_of_token(mem, p.L)
    nb = mem.shape[0]
    qn, kn = to_np(inp["q"]), to_np(inp["k"])
    mask, shat, stats = otok.select_tokens_all_heads(qn, oracle.block_means(kn, mem), 0.25, blk)
    del kn
    print(f"  oracle done: pool {p.L}x{nb}, k* {[s['k'] for s in stats]}", flush=True)
    d = {x: inp[x].to(DEV) for x in ("q", "k", "v", "do")}
    _, kp = vmoba_partition_pool(p, d["q"], d["k"])
    sel = vmoba_select_tokens(p, d["q"], kp, 0.25)
    torch.cuda.synchronize()
    gm = bits_to_bool(sel.token_mask, nb)
    bad = exempt = 0
    for h in range(p.heads):
        v = stats[h]["v"]
        diff = gm[h] != mask[0, h]
        near = np.abs(shat[0, h] - v) <= 1e-4 * v
        bad += int((diff & ~near).sum())
        exempt += int((diff & near).sum())
    print(f"  mask mismatches {bad} exempt {exempt} density {gm.mean():.4f}", flush=True)
    assert bad == 0
    del shat
    union = otok.union_block_mask(mask, mem)
    rp, ci, cp, ri = csr_to_device(union, DEV)
    bits = bool_to_bits(mask[0]).to(DEV)
    o, lse = vmoba_token_attn_fwd(p, d["q"], d["k"], d["v"], rp, ci, bits)
    dq, dk, dv = vmoba_token_attn_bwd(p, d["q"], d["k"], d["v"], o, lse, d["do"], rp, ci, cp,
                                      ri, bits)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    q, k, v, do = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    on, ln, dqn = o.float().cpu().numpy(), lse.cpu().numpy(), dq.cpu().numpy()
    for h in range(p.heads):
        rows = np.sort(rng.choice(p.L, 48, replace=False))
        got = otok.sampled_token_rows(q, k, v, do, mask, mem, blk, 0, h, rows)
        for x, r in zip(rows, got):
            assert np.abs(on[0, x, h] - r["o"]).max() <= TOL
            assert abs(ln[0, h, x] - r["lse"]) <= TOL
            assert np.abs(dqn[0, x, h] - r["dq"]).max() <= TOL
    # sum_y dV_y = sum_x dO_x and sum_y dK_y = 0 (fp64 sums of the fp32 gradients)
    dvs = dv.double().sum(dim=1).cpu().numpy()
    dos = inp["do"].double().sum(dim=1).numpy()
    dks = dk.double().sum(dim=1).cpu().numpy()
    scale = np.abs(dos).max()
    assert np.abs(dvs - dos).max() <= 1e-3 * scale
    assert np.abs(dks).max() <= 1e-3 * max(1.0, np.abs(dk.double().cpu().numpy()).sum(axis=1).max())
