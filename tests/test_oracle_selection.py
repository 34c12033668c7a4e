"""Pins of the oracle's scores, normalisation and threshold selection (CPU only).

papernotes 关键设计 2 (global pool of query-block x key-block similarities per
head) and 关键设计 3 (k = min{k' : sum of the k' largest normalised
similarities >= tau}; the kept token sparsity is always below tau).
"""

import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_pool(rng, nb, d=8, scale=1.0):
    return (rng.standard_normal((1, 1, nb, d)) * scale,
            rng.standard_normal((1, 1, nb, d)) * scale)


def test_block_score_is_mean_of_token_scores():
    # linearity: <mean_i q, mean_j k>/sqrt(d) = mean over token pairs of q.k/sqrt(d)
    rng = np.random.default_rng(3)
    T, H, W, block = 4, 4, 4, (2, 2, 2)
    L, d = 64, 16
    q = rng.standard_normal((1, L, 2, d))
    k = rng.standard_normal((1, L, 2, d))
    mem = oracle.block_members(T, H, W, block)
    s = oracle.block_scores(oracle.block_means(q, mem), oracle.block_means(k, mem))
    for h in range(2):
        tok = q[0, :, h, :] @ k[0, :, h, :].T / np.sqrt(d)      # [L, L]
        for i in range(mem.shape[0]):
            for j in range(mem.shape[0]):
                ref = tok[np.ix_(mem[i], mem[j])].mean()
                assert s[0, h, i, j] == pytest.approx(ref, abs=1e-12)


def test_normalisation_is_softmax_over_whole_head_pool():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((2, 3, 5, 5)) * 3
    shat = oracle.normalise_per_head(s)
    ref = softmax(s.reshape(2, 3, 25), axis=-1).reshape(2, 3, 5, 5)
    np.testing.assert_allclose(shat, ref, rtol=1e-13, atol=0)
    np.testing.assert_allclose(shat.sum(axis=(2, 3)), 1.0, atol=1e-13)
    assert (shat > 0).all()


def test_golden_threshold_example():
    with open(os.path.join(GOLDEN, "threshold_example.json")) as f:
        g = json.load(f)
    s = np.log(np.array(g["exp_scores"], dtype=np.float64))[None, None]
    shat = oracle.normalise_per_head(s)
    np.testing.assert_allclose(shat[0, 0], np.array(g["normalised"]), atol=1e-15)
    for case in g["cases"]:
        r = oracle.threshold_select(shat[0, 0], case["tau"])
        assert r["k"] == case["k"], case
        assert sorted(map(list, zip(*np.nonzero(r["mask"])))) == sorted(case["selected"])


def _brute_min_size(shat_flat, tau):
    n = shat_flat.size
    for size in range(1, n + 1):
        best = max(sum(shat_flat[list(c)]) for c in itertools.combinations(range(n), size))
        if best >= tau:
            return size
    return n


@pytest.mark.parametrize("seed", range(6))
def test_threshold_is_minimal_prefix_by_brute_force(seed):
    # N_b = 4: 16 pairs; brute force over every subset of the pool
    rng = np.random.default_rng(10 + seed)
    qp, kp = _rand_pool(rng, 4, scale=1.5)
    shat = oracle.normalise_per_head(oracle.block_scores(qp, kp))[0, 0]
    flat = shat.reshape(-1)
    for tau in (0.05, 0.25, 0.5, 0.8, 0.97):
        r = oracle.threshold_select(shat, tau)
        k = r["k"]
        assert k == _brute_min_size(flat, tau)
        # the prefix (before the diagonal is added) is the heaviest k-subset
        prefix = set(r["order"][:k].tolist())
        heaviest = max(itertools.combinations(range(16), k),
                       key=lambda c: sum(flat[list(c)]))
        assert prefix == set(heaviest)
        assert sum(flat[list(prefix)]) >= tau
        # token sparsity of the prefix stays below tau (关键设计 3)
        assert (k - 1) / 16 < tau
        # diagonal always kept, nothing else beyond the prefix
        m = r["mask"].copy()
        assert m.diagonal().all()
        extra = {i * 4 + i for i in range(4)} - prefix
        assert m.sum() == k + len(extra)


def test_nested_in_tau_and_tau_one_selects_all():
    rng = np.random.default_rng(5)
    qp, kp = _rand_pool(rng, 12, d=16, scale=2.0)
    shat = oracle.normalise_per_head(oracle.block_scores(qp, kp))[0, 0]
    prev = None
    for tau in np.linspace(0.02, 0.98, 25):
        m = oracle.threshold_select(shat, tau)["mask"]
        if prev is not None:
            assert (m | prev).sum() == m.sum()     # prev subset of m
        prev = m
    assert oracle.threshold_select(shat, 1.0)["mask"].all()


def test_ties_break_by_ascending_linear_index():
    shat = np.full((3, 3), 1.0 / 9)
    r = oracle.threshold_select(shat, 3.5 / 9)   # needs 4 of 9 equal entries
    assert r["k"] == 4
    assert r["order"][:4].tolist() == [0, 1, 2, 3]
    sel = set(zip(*np.nonzero(r["mask"])))
    assert sel == {(0, 0), (0, 1), (0, 2), (1, 0), (1, 1), (2, 2)}


@pytest.mark.parametrize("nb", [1, 5, 17])
def test_token_sparsity_below_tau_on_random_pools(nb):
    rng = np.random.default_rng(nb)
    for _ in range(20):
        qp, kp = _rand_pool(rng, nb, d=32, scale=rng.uniform(0.1, 3))
        shat = oracle.normalise_per_head(oracle.block_scores(qp, kp))[0, 0]
        tau = rng.uniform(0.01, 0.99)
        r = oracle.threshold_select(shat, tau)
        assert (r["k"] - 1) / nb ** 2 < tau
        assert r["k"] <= int(np.ceil(tau * nb * nb))
        assert r["mass"] >= tau


def test_csr_csc_round_trip():
    rng = np.random.default_rng(6)
    mask = rng.random((3, 7, 7)) < 0.3
    rp, ci = oracle.mask_to_csr(mask)
    cp, ri = oracle.mask_to_csc(mask)
    for g in range(3):
        back = np.zeros((7, 7), dtype=bool)
        for i in range(7):
            cols = ci[g, rp[g, i]:rp[g, i + 1]]
            assert (np.diff(cols) > 0).all()
            back[i, cols] = True
        assert (back == mask[g]).all()
        back[:] = False
        for j in range(7):
            rows = ri[g, cp[g, j]:cp[g, j + 1]]
            assert (np.diff(rows) > 0).all()
            back[rows, j] = True
        assert (back == mask[g]).all()
