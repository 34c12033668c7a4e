"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle, compare."""

import numpy as np
import torch

import oracle
from block_sparse_attention_layer_amd import (
    Problem, vmoba_partition_pool, vmoba_select, vmoba_sparse_attn_bwd,
    vmoba_sparse_attn_fwd)

# tolerances (max-abs) for attention outputs and gradients
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
# selection: pairs whose oracle score lies within this of the oracle cutoff are exempt
MASK_WINDOW = 1e-5


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def masks_from_csr(row_ptr, col_idx, nb):
    rp = row_ptr.cpu().numpy()
    ci = col_idx.cpu().numpy()
    G = rp.shape[0]
    m = np.zeros((G, nb, nb), dtype=bool)
    for g in range(G):
        for i in range(nb):
            m[g, i, ci[g, rp[g, i]:rp[g, i + 1]]] = True
    return m


def masks_from_csc(col_ptr, row_idx, nb):
    return np.swapaxes(masks_from_csr(col_ptr, row_idx, nb), -1, -2)


def csr_to_device(mask, device):
    """Oracle block mask [B, Hh, Nb, Nb] -> device CSR and CSC (oracle-side conversion)."""
    G = mask.shape[0] * mask.shape[1]
    m = mask.reshape(G, mask.shape[2], mask.shape[3])
    rp, ci = oracle.mask_to_csr(m)
    cp, ri = oracle.mask_to_csc(m)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return f(rp), f(ci), f(cp), f(ri)


def compare_masks(gpu_mask, ora_mask, shat, stats, window=MASK_WINDOW):
    """Mismatches outside the cutoff window; returns (n_mismatch, n_exempt_diffs)."""
    B, Hh, nb, _ = ora_mask.shape
    gm = gpu_mask.reshape(B, Hh, nb, nb)
    bad = exempt = 0
    for b in range(B):
        for h in range(Hh):
            v = stats[b * Hh + h]["v"]
            diff = gm[b, h] != ora_mask[b, h]
            near = np.abs(shat[b, h] - v) <= window
            bad += int((diff & ~near).sum())
            exempt += int((diff & near).sum())
    return bad, exempt


def problem_for(cfg, spec, dtype, batch=None, heads=None, head_dim=None):
    return Problem(batch or cfg["batch"], heads or cfg["heads"], head_dim or cfg["head_dim"],
                   cfg["T"], cfg["H"], cfg["W"], spec.layer_idx, tuple(spec.block), dtype)


def gpu_pool_select(p, q, k, tau, want_scores=False):
    qp, kp = vmoba_partition_pool(p, q, k)
    sel = vmoba_select(p, qp, kp, tau, want_scores=want_scores)
    torch.cuda.synchronize()
    return qp, kp, sel


def max_err(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
