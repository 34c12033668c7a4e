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


import test_oracle_selection_modes as t_modes


def test_modes_pins_pass_unmutated():
    assert not _fails(t_modes.test_golden_local_and_topk_examples)
    assert not _fails(t_modes.test_row_normalisation_is_row_softmax)


def test_local_pool_normalised_over_the_head_is_caught(monkeypatch):
    # planted slip: the local rule fed head-normalised scores (the global pool's shares)
    monkeypatch.setattr(oracle, "normalise_per_row",
                        lambda s: sel.normalise_per_head(np.asarray(s, float)[None, None])[0, 0]
                        if np.ndim(s) == 2 else sel.normalise_per_head(s))
    assert _fails(t_modes.test_golden_local_and_topk_examples)


def test_topk_off_by_one_is_caught(monkeypatch):
    orig = sel.topk_select
    monkeypatch.setattr(oracle, "topk_select", lambda shat, k: orig(shat, k + 1))
    assert _fails(t_modes.test_topk_global_keeps_a_dominant_set_of_exactly_k, 0)


def test_local_strict_inequality_is_caught(monkeypatch):
    orig = sel.local_select

    def strict(shat_rows, tau=None, k=None):
        return orig(shat_rows, tau=None if tau is None else np.nextafter(tau, 2.0), k=k)
    monkeypatch.setattr(oracle, "local_select", strict)
    assert _fails(t_modes.test_golden_local_and_topk_examples)


def test_transposed_head_split_in_dit_block_is_caught(monkeypatch):
    """Channels grouped into heads as [d, Hh] instead of [Hh, d]."""
    import test_oracle_dit as t_dit
    from oracle import dit as odit
    orig = odit._OracleAttention.apply

    def wrong(q, k, v, members, mask):
        B, L, Hh, d = q.shape
        to = lambda t: t.reshape(B, L, d, Hh).transpose(2, 3).contiguous()
        a = orig(to(q), to(k), to(v), members, mask)
        return a.transpose(2, 3).reshape(B, L, Hh, d)

    assert not _fails(t_dit.test_heads_with_zero_query_key_average_selected_values, 2,
                      (1, 2, 2))
    monkeypatch.setattr(odit._OracleAttention, "apply", wrong)
    assert _fails(t_dit.test_heads_with_zero_query_key_average_selected_values, 2, (1, 2, 2))


def test_token_pool_normalised_per_token_is_caught(monkeypatch):
    import test_oracle_tokens as t_tok
    from oracle import tokens as otok

    def per_token(s):
        e = np.exp(s - s.max(axis=-1, keepdims=True))
        return e / e.sum(axis=-1, keepdims=True)
    assert not _fails(t_tok.test_pool_normalisation_sums_to_one)
    monkeypatch.setattr(otok, "normalise_token_pool", per_token)
    assert _fails(t_tok.test_pool_normalisation_sums_to_one)


def test_token_ties_by_descending_index_are_caught(monkeypatch):
    import test_oracle_tokens as t_tok
    from oracle import tokens as otok

    def desc_ties(vals, tau=None, k=None):
        vals = np.asarray(vals, float)
        n = vals.size
        order = (n - 1 - np.argsort(-vals[::-1], kind="stable"))
        hit = np.nonzero(np.cumsum(vals[order]) >= tau)[0]
        return order, (int(hit[0]) + 1 if hit.size else n)
    assert not _fails(t_tok.test_hand_worked_example_with_ties)
    monkeypatch.setattr(otok, "_ordered_prefix", desc_ties)
    assert _fails(t_tok.test_hand_worked_example_with_ties)


def test_token_forced_pair_of_wrong_block_is_caught(monkeypatch):
    import test_oracle_tokens as t_tok
    from oracle import tokens as otok
    orig = otok.token_select

    def wrong_diag(shat, tau, blk_of_tok):
        L, nb = np.asarray(shat).shape
        return orig(shat, tau, np.arange(L) % nb)     # token index mod N_b, not its block
    assert not _fails(t_tok.test_prefix_invariants, 1)
    monkeypatch.setattr(otok, "token_select", wrong_diag)
    assert _fails(t_tok.test_prefix_invariants, 1)


def test_token_pool_temperature_slip_is_caught(monkeypatch):
    """A scale inside the token-pool softmax still sums to one; the scipy pin sees it."""
    import test_oracle_tokens as t_tok
    from oracle import tokens as otok
    orig = otok.normalise_token_pool

    def hot(s):
        return orig(np.asarray(s, float) / 0.9)
    assert not _fails(t_tok.test_pool_normalisation_is_scipy_softmax_over_flattened_pool)
    monkeypatch.setattr(otok, "normalise_token_pool", hot)
    assert not _fails(t_tok.test_pool_normalisation_sums_to_one)
    assert _fails(t_tok.test_pool_normalisation_is_scipy_softmax_over_flattened_pool)
