"""Pins of the oracle's token-granular query pool (CPU only).

- scores: the token-to-block score equals the mean of the token-to-token scores over the
  key block (by linearity of the block mean), computed here by explicit loops;
- normalisation: every head's pool sums to one, and equals scipy's softmax over the
  head's flattened L * N_b pool (shift-invariant per head, heads independent);
- threshold: brute force over every subset of a 16-entry pool finds the same minimal
  count; minimality, the ceil(tau L N_b) bound and nestedness in tau; a hand-worked
  example whose cut falls inside a run of equal values (ties by ascending index);
- the forced pairs: every token keeps its own block;
- attention: tau = 1 selects every pair and gives torch's fp64 scaled_dot_product_attention
  and logsumexp; a token mask constant over each query block gives the block-sparse
  attention of that block mask; sampled rows equal the L x L form.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import tokens as otok


def _setup(T=2, H=4, W=4, block=(1, 2, 2), layer=2, heads=2, d=8, seed=0):
    rng = np.random.default_rng(seed)
    L = T * H * W
    q = rng.standard_normal((1, L, heads, d))
    k = rng.standard_normal((1, L, heads, d))
    v = rng.standard_normal((1, L, heads, d))
    do = rng.standard_normal((1, L, heads, d))
    oracle.check_partition(T, H, W, layer, block)
    mem = oracle.block_members(T, H, W, block)
    blk = oracle.block_of_token(mem, L)
    return q, k, v, do, mem, blk


def test_token_scores_are_means_of_token_dot_products():
    q, k, v, do, mem, blk = _setup()
    kp = oracle.block_means(k, mem)
    s = otok.token_scores(q, kp)
    d = q.shape[-1]
    for h in range(q.shape[2]):
        for x in range(q.shape[1]):
            for j in range(mem.shape[0]):
                want = np.mean([q[0, x, h] @ k[0, y, h] for y in mem[j]]) / math.sqrt(d)
                assert abs(s[0, h, x, j] - want) <= 1e-12


def test_pool_normalisation_sums_to_one():
    q, k, v, do, mem, blk = _setup()
    shat = otok.normalise_token_pool(otok.token_scores(q, oracle.block_means(k, mem)))
    assert (shat >= 0).all()
    assert np.abs(shat.sum(axis=(2, 3)) - 1.0).max() <= 1e-12


def test_pool_normalisation_is_scipy_softmax_over_flattened_pool():
    """Against scipy's softmax over each head's L * N_b entries (a library routine): a
    temperature, a scale, a per-row or per-column normaliser or a mixed-up head would
    each differ.  Scores spread over [-40, 40] so exp without the max shift overflows
    nowhere but a wrong scale is far off."""
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    B, Hh, L, nb = 2, 3, 12, 5
    s = rng.uniform(-40.0, 40.0, (B, Hh, L, nb))
    s[1, 2] *= 0.01                       # one nearly uniform head
    got = otok.normalise_token_pool(s)
    want = softmax(s.reshape(B, Hh, L * nb), axis=-1).reshape(B, Hh, L, nb)
    assert np.abs(got - want).max() <= 1e-14
    assert np.abs(got[1, 2] - 1.0 / (L * nb)).max() <= 0.5 / (L * nb)
    # shift invariance per head, and no coupling between heads
    s2 = s.copy()
    s2[0, 1] += 123.0
    got2 = otok.normalise_token_pool(s2)
    assert np.abs(got2 - got).max() <= 1e-14


@pytest.mark.parametrize("tau", [0.1, 0.25, 0.5, 0.8])
def test_brute_force_minimal_count(tau):
    rng = np.random.default_rng(5)
    L, nb = 8, 2
    shat = rng.random((L, nb)) ** 3
    shat /= shat.sum()
    r = otok.token_select(shat, tau, np.zeros(L, dtype=int))
    flat = shat.reshape(-1)
    best = None
    for size in range(1, flat.size + 1):
        if any(flat[list(c)].sum() >= tau for c in itertools.combinations(range(flat.size), size)):
            best = size
            break
    assert r["k"] == best


@pytest.mark.parametrize("seed", [1, 2])
def test_prefix_invariants(seed):
    q, k, v, do, mem, blk = _setup(seed=seed)
    kp = oracle.block_means(k, mem)
    prev = None
    for tau in (0.05, 0.25, 0.5, 0.9):
        mask, shat, stats = otok.select_tokens_all_heads(q, kp, tau, blk)
        L, nb = shat.shape[2], shat.shape[3]
        for h, st in enumerate(stats):
            assert st["mass"] >= tau and st["mass"] - st["v"] < tau
            assert st["k"] <= math.ceil(tau * L * nb)
            assert mask[0, h, np.arange(L), blk].all()         # own block kept
        if prev is not None:
            assert (mask | ~prev).all() and (prev <= mask).all()   # nested in tau
        prev = mask


def test_hand_worked_example_with_ties():
    # 4 tokens, 2 blocks (tokens 0, 1 in block 0; 2, 3 in block 1); masses m[x][j]:
    m = np.array([[4.0, 1.0], [2.0, 1.0], [1.0, 8.0], [1.0, 1.0]])
    shat = m / m.sum()                       # total 19
    blk = np.array([0, 0, 1, 1])
    # tau 0.5: 8 then 4 reach 12/19 >= 0.5 -> (2,1), (0,0); plus own blocks
    r = otok.token_select(shat, 0.5, blk)
    assert r["k"] == 2
    assert (r["mask"] == np.array([[1, 0], [1, 0], [0, 1], [0, 1]], bool)).all()
    # tau 0.75 (14.25 of 19): 8, 4, 2, then one mass-1 entry; of the five tied ones the
    # lowest linear index x*2 + j is (0, 1)
    r = otok.token_select(shat, 0.75, blk)
    assert r["k"] == 4 and abs(r["v"] - 1 / 19) < 1e-15
    assert (r["mask"] == np.array([[1, 1], [1, 0], [0, 1], [0, 1]], bool)).all()


def test_tau_one_is_full_attention():
    q, k, v, do, mem, blk = _setup()
    mask, _, _ = otok.select_tokens_all_heads(q, oracle.block_means(k, mem), 1.0, blk)
    assert mask.all()
    o, lse = otok.token_attention_fwd(q, k, v, mask, blk)
    tq, tk, tv = (torch.from_numpy(t).permute(0, 2, 1, 3) for t in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3)
    assert np.abs(o - ref.numpy()).max() <= 1e-12
    z = tq @ tk.transpose(-1, -2) / math.sqrt(q.shape[-1])
    assert np.abs(lse - torch.logsumexp(z, dim=-1).numpy()).max() <= 1e-12


def test_block_constant_token_mask_is_block_attention():
    q, k, v, do, mem, blk = _setup()
    rng = np.random.default_rng(9)
    nb = mem.shape[0]
    bm = rng.random((1, q.shape[2], nb, nb)) < 0.4
    bm[:, :, np.arange(nb), np.arange(nb)] = True
    tm = bm[:, :, blk, :]                    # token x takes its block's row
    assert (otok.union_block_mask(tm, mem) == bm).all()
    o1, l1 = otok.token_attention_fwd(q, k, v, tm, blk)
    o2, l2 = oracle.sparse_attention_fwd(q, k, v, mem, bm)
    assert np.abs(o1 - o2).max() <= 1e-12 and np.abs(l1 - l2).max() <= 1e-12
    g1 = otok.token_attention_bwd(q, k, v, o1, l1, do, tm, blk)
    g2 = oracle.sparse_attention_bwd(q, k, v, o2, l2, do, mem, bm)
    for a, b in zip(g1, g2):
        assert np.abs(a - b).max() <= 1e-12


def test_union_and_sampled_rows():
    q, k, v, do, mem, blk = _setup()
    kp = oracle.block_means(k, mem)
    mask, _, _ = otok.select_tokens_all_heads(q, kp, 0.3, blk)
    u = otok.union_block_mask(mask, mem)
    for h in range(q.shape[2]):
        for i in range(mem.shape[0]):
            want = np.zeros(mem.shape[0], bool)
            for x in mem[i]:
                want |= mask[0, h, x]
            assert (u[0, h, i] == want).all()
    o, lse = otok.token_attention_fwd(q, k, v, mask, blk)
    dq, _, _ = otok.token_attention_bwd(q, k, v, o, lse, do, mask, blk)
    rows = [0, 5, 17, 31]
    for h in range(q.shape[2]):
        got = otok.sampled_token_rows(q, k, v, do, mask, mem, blk, 0, h, rows)
        for x, r in zip(rows, got):
            assert np.abs(r["o"] - o[0, x, h]).max() <= 1e-12
            assert abs(r["lse"] - lse[0, h, x]) <= 1e-12
            assert np.abs(r["dq"] - dq[0, x, h]).max() <= 1e-12
