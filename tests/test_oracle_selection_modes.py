"""Pins of the oracle's other selection strategies (CPU only).

paperlayer §4.4 (Table 3) and the papernotes ablation table compare the default
threshold + global selection with top-k + global, threshold + local and top-k + local
(the last being MoBA's rule).  Each pin below checks a property that a plausible slip
would break: the row normalisation, the dominance order of the kept set, minimality of
each row's threshold prefix (also by brute force), exact counts for top-k, independence
of the rows in the local modes, and hand-derived examples.
"""

import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ints(rng, shape, lo=-3, hi=3):
    # integer scores: many exact ties, so the tie rule is exercised
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def _dominates(vals, kept):
    """Every kept entry precedes every other one in (value desc, index asc) order."""
    idx = np.arange(vals.size)
    for a in idx[kept]:
        for b in idx[~kept]:
            if not (vals[a] > vals[b] or (vals[a] == vals[b] and a < b)):
                return False
    return True


def test_row_normalisation_is_row_softmax():
    rng = np.random.default_rng(11)
    s = rng.standard_normal((2, 3, 6, 6)) * 4
    shat = oracle.normalise_per_row(s)
    np.testing.assert_allclose(shat, softmax(s, axis=-1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(shat.sum(axis=-1), 1.0, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_topk_global_keeps_a_dominant_set_of_exactly_k(seed):
    rng = np.random.default_rng(seed)
    nb = 4
    shat = _ints(rng, (nb, nb))
    for k in range(0, nb * nb + 3):
        r = oracle.topk_select(shat, k)
        kept = np.zeros(nb * nb, bool)
        kept[r["order"][:r["k"]]] = True
        assert kept.sum() == min(k, nb * nb)
        assert _dominates(shat.reshape(-1), kept)
        expect = kept.reshape(nb, nb).copy()
        expect[np.arange(nb), np.arange(nb)] = True
        np.testing.assert_array_equal(r["mask"], expect)


@pytest.mark.parametrize("seed", range(4))
def test_topk_global_at_kstar_equals_threshold(seed):
    # the threshold rule keeps the k* largest pairs; top-k at that k keeps the same set
    rng = np.random.default_rng(20 + seed)
    qp, kp = rng.standard_normal((1, 1, 7, 8)), rng.standard_normal((1, 1, 7, 8))
    shat = oracle.normalise_per_head(oracle.block_scores(qp, kp))[0, 0]
    for tau in (0.1, 0.25, 0.5, 0.9):
        t = oracle.threshold_select(shat, tau)
        np.testing.assert_array_equal(oracle.topk_select(shat, t["k"])["mask"], t["mask"])


@pytest.mark.parametrize("seed", range(6))
def test_threshold_local_is_minimal_prefix_by_brute_force(seed):
    rng = np.random.default_rng(40 + seed)
    nb = 4
    s = _ints(rng, (nb, nb), -2, 2) * 0.7
    shat = oracle.normalise_per_row(s)
    for tau in (0.2, 0.25, 0.5, 0.75, 0.99):
        r = oracle.local_select(shat, tau=tau)
        for i in range(nb):
            row = shat[i]
            # smallest subset size whose mass reaches tau, over all 2^nb subsets
            best = min(len(c) for n in range(nb + 1) for c in itertools.combinations(range(nb), n)
                       if row[list(c)].sum() >= tau) if row.sum() >= tau else nb
            assert r["row_k"][i] == best
            kept = np.zeros(nb, bool)
            kept[np.argsort(-row, kind="stable")[:best]] = True
            assert _dominates(row, kept)
            expect = kept.copy()
            expect[i] = True
            np.testing.assert_array_equal(r["mask"][i], expect)


def test_threshold_local_tau_one_and_nestedness():
    rng = np.random.default_rng(7)
    shat = oracle.normalise_per_row(rng.standard_normal((9, 9)) * 2)
    assert oracle.local_select(shat, tau=1.0)["mask"].all()
    prev = None
    for tau in (0.05, 0.15, 0.25, 0.5, 0.8):
        m = oracle.local_select(shat, tau=tau)["mask"]
        if prev is not None:
            assert (m | prev == m).all()      # a larger tau keeps a superset
        prev = m
    for i in range(9):                         # each row's prefix reaches tau
        r = oracle.local_select(shat, tau=0.3)
        assert r["row_mass"][i] >= 0.3


@pytest.mark.parametrize("seed", range(4))
def test_topk_local_counts_and_dominance(seed):
    rng = np.random.default_rng(60 + seed)
    nb = 6
    shat = oracle.normalise_per_row(_ints(rng, (nb, nb)))
    for k in (0, 1, 2, 5, 6, 9):
        r = oracle.local_select(shat, k=k)
        for i in range(nb):
            assert r["row_k"][i] == min(k, nb)
            kept = np.zeros(nb, bool)
            kept[np.argsort(-shat[i], kind="stable")[:min(k, nb)]] = True
            assert _dominates(shat[i], kept)
            assert r["mask"][i].sum() == min(k, nb) + (0 if kept[i] else 1)


@pytest.mark.parametrize("mode,kw", [("threshold_local", {"tau": 0.3, "k": None}),
                                     ("topk_local", {"tau": None, "k": 3})])
def test_local_rows_are_independent(mode, kw):
    # changing one query block's pooled vector changes only that row of a local selection
    rng = np.random.default_rng(5)
    qp, kp = rng.standard_normal((1, 2, 8, 16)), rng.standard_normal((1, 2, 8, 16))
    m0, _, _ = oracle.select_all_heads(qp, kp, mode=mode, **kw)
    qp2 = qp.copy()
    qp2[0, :, 3] = rng.standard_normal((2, 16)) * 5
    m1, _, _ = oracle.select_all_heads(qp2, kp, mode=mode, **kw)
    rows = [i for i in range(8) if i != 3]
    np.testing.assert_array_equal(m0[:, :, rows], m1[:, :, rows])


def test_global_threshold_couples_rows():
    # the global pool is shared: one row with very large scores takes the mass of others
    rng = np.random.default_rng(6)
    qp, kp = rng.standard_normal((1, 1, 8, 16)), rng.standard_normal((1, 1, 8, 16))
    m0, _, _ = oracle.select_all_heads(qp, kp, 0.25)
    qp2 = qp.copy()
    qp2[0, 0, 3] = kp[0, 0, 5] * 40            # row 3 aligns strongly with key block 5
    m1, _, _ = oracle.select_all_heads(qp2, kp, 0.25)
    others = [i for i in range(8) if i != 3]
    assert m1[0, 0, others].sum() < m0[0, 0, others].sum()


def test_golden_local_and_topk_examples():
    with open(os.path.join(GOLDEN, "local_selection_example.json")) as f:
        g = json.load(f)
    s = np.log(np.array(g["exp_scores"], dtype=np.float64))
    np.testing.assert_allclose(oracle.normalise_per_row(s), np.array(g["row_normalised"]),
                               atol=1e-15)
    def as_pairs(mask):
        return sorted([list(map(int, p)) for p in zip(*np.nonzero(mask))])
    for case in g["threshold_local"]:
        r = oracle.local_select(oracle.normalise_per_row(s), tau=case["tau"])
        assert r["row_k"].tolist() == case["row_k"], case["why"]
        assert as_pairs(r["mask"]) == case["selected"], case["why"]
    for case in g["topk_local"]:
        r = oracle.local_select(oracle.normalise_per_row(s), k=case["k"])
        assert as_pairs(r["mask"]) == case["selected"], case["why"]
    for case in g["topk_global"]:
        shat = oracle.normalise_per_head(s[None, None])[0, 0]
        r = oracle.topk_select(shat, case["k"])
        assert as_pairs(r["mask"]) == case["selected"], case["why"]


def test_select_all_heads_modes_agree_with_single_head_functions():
    rng = np.random.default_rng(9)
    qp, kp = rng.standard_normal((2, 2, 6, 8)), rng.standard_normal((2, 2, 6, 8))
    s = oracle.block_scores(qp, kp)
    for mode, kw in [("topk_global", {"tau": None, "k": 7}),
                     ("threshold_local", {"tau": 0.4, "k": None}),
                     ("topk_local", {"tau": None, "k": 2})]:
        mask, shat, stats = oracle.select_all_heads(qp, kp, mode=mode, **kw)
        for b in range(2):
            for h in range(2):
                if mode == "topk_global":
                    ref = oracle.topk_select(oracle.normalise_per_head(s)[b, h], 7)["mask"]
                else:
                    ref = oracle.local_select(oracle.normalise_per_row(s)[b, h],
                                              tau=kw["tau"], k=kw["k"])["mask"]
                np.testing.assert_array_equal(mask[b, h], ref)
                assert stats[b * 2 + h]["nnz"] == int(ref.sum())
    with pytest.raises(ValueError):
        oracle.select_all_heads(qp, kp, 0.25, mode="bogus")
