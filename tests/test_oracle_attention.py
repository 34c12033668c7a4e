"""Pins of the oracle's attention forward and backward (CPU only).

With every block selected the layer is full attention; with a block mask it is
masked attention.  Both are compared with torch's scaled_dot_product_attention
in fp64 (a library routine), gradients with torch.autograd of that routine and
with central finite differences.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

T, H, W, BLOCK = 2, 4, 4, (1, 2, 2)      # 32 tokens, 8 blocks of 4


def _inputs(seed, B=1, Hh=2, d=8):
    rng = np.random.default_rng(seed)
    L = T * H * W
    shp = (B, L, Hh, d)
    return [rng.standard_normal(shp) for _ in range(4)]


def _sdpa(q, k, v, tok_mask):
    # torch wants [B, Hh, L, d]; mask True = attend
    tq, tk, tv = [torch.tensor(x).permute(0, 2, 1, 3) for x in (q, k, v)]
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(tok_mask))
    return o.permute(0, 2, 1, 3).numpy()


def _tok_mask(block_mask, blk):
    B, Hh = block_mask.shape[:2]
    return np.stack([np.stack([oracle.token_mask(block_mask[b, h], blk)
                               for h in range(Hh)]) for b in range(B)])


def _setup(seed, density):
    mem = oracle.block_members(T, H, W, BLOCK)
    blk = oracle.block_of_token(mem, T * H * W)
    rng = np.random.default_rng(100 + seed)
    nb = mem.shape[0]
    bm = rng.random((1, 2, nb, nb)) < density
    bm |= np.eye(nb, dtype=bool)
    return mem, blk, bm


@pytest.mark.parametrize("seed", [0, 1])
def test_all_blocks_is_full_attention(seed):
    q, k, v, _ = _inputs(seed)
    mem, blk, _ = _setup(seed, 1.0)
    nb = mem.shape[0]
    full = np.ones((1, 2, nb, nb), dtype=bool)
    o, lse = oracle.sparse_attention_fwd(q, k, v, mem, full)
    tq, tk, tv = [torch.tensor(x).permute(0, 2, 1, 3) for x in (q, k, v)]
    ref = F.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    # textbook softmax(Q K^T / sqrt(d)) V
    d = q.shape[-1]
    for h in range(2):
        z = q[0, :, h] @ k[0, :, h].T / np.sqrt(d)
        p = np.exp(z - z.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(o[0, :, h], p @ v[0, :, h], atol=1e-12)
        np.testing.assert_allclose(lse[0, h], torch.logsumexp(torch.tensor(z), 1).numpy(),
                                   atol=1e-12)


@pytest.mark.parametrize("seed,density", [(0, 0.3), (1, 0.5), (2, 0.0)])
def test_block_sparse_matches_masked_sdpa_and_literal_form(seed, density):
    q, k, v, _ = _inputs(seed)
    mem, blk, bm = _setup(seed, density)
    o, lse = oracle.sparse_attention_fwd(q, k, v, mem, bm)
    tm = _tok_mask(bm, blk)
    np.testing.assert_allclose(o, _sdpa(q, k, v, tm), atol=1e-12)
    o2, lse2 = oracle.dense_masked_attention_fwd(q, k, v, tm)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-12)
    d = q.shape[-1]
    z = torch.tensor(np.einsum("blhd,bmhd->bhlm", q, k) / np.sqrt(d))
    z = z.masked_fill(~torch.tensor(tm), -float("inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(z, -1).numpy(), atol=1e-12)


@pytest.mark.parametrize("seed,density", [(0, 0.3), (3, 0.6), (4, 1.0)])
def test_backward_matches_autograd(seed, density):
    q, k, v, do = _inputs(seed)
    mem, blk, bm = _setup(seed, density)
    o, lse = oracle.sparse_attention_fwd(q, k, v, mem, bm)
    dq, dk, dv = oracle.sparse_attention_bwd(q, k, v, o, lse, do, mem, bm)
    tm = torch.tensor(_tok_mask(bm, blk))
    tq, tk, tv = [torch.tensor(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v)]
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), atol=1e-11)
    # literal dense form agrees too
    dq2, dk2, dv2 = oracle.dense_masked_attention_bwd(q, k, v, o, lse, do, tm.numpy())
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_backward_central_differences():
    q, k, v, do = _inputs(7, Hh=1, d=4)
    mem, blk, bm = _setup(7, 0.4)

    def loss(qq, kk, vv):
        o, _ = oracle.sparse_attention_fwd(qq, kk, vv, mem, bm)
        return float((o * do).sum())

    o, lse = oracle.sparse_attention_fwd(q, k, v, mem, bm)
    grads = oracle.sparse_attention_bwd(q, k, v, o, lse, do, mem, bm)
    rng = np.random.default_rng(0)
    eps = 1e-6
    for which, g in enumerate(grads):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in q.shape)
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            dn = loss(*args)
            assert g[idx] == pytest.approx((up - dn) / (2 * eps), abs=1e-6)


def test_sampled_rows_and_key_blocks_match_full_computation():
    q, k, v, do = _inputs(8)
    mem, blk, bm = _setup(8, 0.35)
    o, lse = oracle.sparse_attention_fwd(q, k, v, mem, bm)
    dq, dk, dv = oracle.sparse_attention_bwd(q, k, v, o, lse, do, mem, bm)
    rows = np.array([0, 5, 17, 31])
    for h in range(2):
        r = oracle.sampled_query_rows(q, k, v, do, mem, blk, bm, 0, h, rows)
        np.testing.assert_allclose(r["o"], o[0, rows, h], atol=1e-12)
        np.testing.assert_allclose(r["lse"], lse[0, h, rows], atol=1e-12)
        np.testing.assert_allclose(r["dq"], dq[0, rows, h], atol=1e-12)
        for j in (0, 3, 7):
            gk, gv = oracle.sampled_key_block_grads(q, k, v, do, mem, bm, 0, h, j)
            np.testing.assert_allclose(gk, dk[0, mem[j], h], atol=1e-12)
            np.testing.assert_allclose(gv, dv[0, mem[j], h], atol=1e-12)


def test_layer_end_to_end_at_tau_one_is_full_attention():
    q, k, v, do = _inputs(9)
    out = oracle.oracle_layer(q, k, v, T, H, W, 2, BLOCK, 1.0, do=do)
    assert out["mask"].all()
    tq, tk, tv = [torch.tensor(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v)]
    ref = F.scaled_dot_product_attention(tq, tk, tv)
    ref.backward(torch.tensor(do).permute(0, 2, 1, 3))
    np.testing.assert_allclose(out["o"], ref.detach().permute(0, 2, 1, 3).numpy(), atol=1e-12)
    np.testing.assert_allclose(out["dk"], tk.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11)
