"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case patches one oracle function with a plausible slip (a dropped term, a
wrong sign or index, a transposed operand, '>' for '>=') and checks that the
pin guarding it now fails.  Mistakes are planted in the oracle only.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as att, selection as sel, pooling as pool

import test_oracle_attention as t_att
import test_oracle_pooling as t_pool
import test_oracle_selection as t_sel


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_pins_pass_unmutated():
    assert not _fails(t_sel.test_block_score_is_mean_of_token_scores)
    assert not _fails(t_sel.test_golden_threshold_example)


def test_dropped_score_scale_is_caught(monkeypatch):
    bad = lambda qp, kp: np.matmul(np.asarray(qp, float), np.swapaxes(np.asarray(kp, float), -1, -2))
    monkeypatch.setattr(sel, "block_scores", bad)
    monkeypatch.setattr(oracle, "block_scores", bad)
    assert _fails(t_sel.test_block_score_is_mean_of_token_scores)


def test_strict_inequality_is_caught(monkeypatch):
    orig = sel.threshold_select

    def strict(shat, tau):
        r = orig(shat, np.nextafter(tau, 2.0))   # behaves like "> tau"
        return r
    monkeypatch.setattr(oracle, "threshold_select", strict)
    assert _fails(t_sel.test_golden_threshold_example)


def test_ascending_sort_is_caught(monkeypatch):
    def ascending(shat, tau):
        shat = np.asarray(shat, float)
        nb = shat.shape[0]
        flat = shat.reshape(-1)
        order = np.argsort(flat, kind="stable")
        csum = np.cumsum(flat[order])
        k = int(np.nonzero(csum >= tau)[0][0]) + 1
        m = np.zeros(nb * nb, bool)
        m[order[:k]] = True
        m = m.reshape(nb, nb)
        m[np.arange(nb), np.arange(nb)] = True
        return {"mask": m, "k": k, "v": float(flat[order][k - 1]),
                "mass": float(csum[k - 1]), "order": order}
    monkeypatch.setattr(oracle, "threshold_select", ascending)
    assert _fails(t_sel.test_threshold_is_minimal_prefix_by_brute_force, 0)


def test_mean_divisor_off_by_one_is_caught(monkeypatch):
    orig = pool.block_means
    monkeypatch.setattr(oracle, "block_means",
                        lambda x, m: orig(x, m) * m.shape[1] / (m.shape[1] - 1))
    assert _fails(t_pool.test_block_means_match_masked_numpy_mean)


def test_transposed_attention_operand_is_caught(monkeypatch):
    orig = att.sparse_attention_fwd
    monkeypatch.setattr(oracle, "sparse_attention_fwd",
                        lambda q, k, v, mem, bm: orig(k, q, v, mem, bm))
    assert _fails(t_att.test_all_blocks_is_full_attention, 0)


def test_missing_delta_term_is_caught(monkeypatch):
    def bad_bwd(q, k, v, o, lse, do, mem, bm):
        # planted slip: delta term dropped (o replaced by zeros)
        return att.sparse_attention_bwd(q, k, v, np.zeros_like(np.asarray(o, float)),
                                        lse, do, mem, bm)
    monkeypatch.setattr(oracle, "sparse_attention_bwd", bad_bwd)
    assert _fails(t_att.test_backward_matches_autograd, 0, 0.3)


def test_block_mask_transposed_is_caught(monkeypatch):
    orig = att.sparse_attention_fwd
    monkeypatch.setattr(oracle, "sparse_attention_fwd",
                        lambda q, k, v, mem, bm: orig(q, k, v, mem, np.swapaxes(bm, -1, -2)))
    assert _fails(t_att.test_block_sparse_matches_masked_sdpa_and_literal_form, 0, 0.3)
