"""Pins of the oracle's block means (CPU only).  papernotes 关键设计 1: B = mean(K')."""

import numpy as np
import pytest

import oracle


def _members(T, H, W, block):
    return oracle.block_members(T, H, W, block)


def test_block_means_match_masked_numpy_mean():
    rng = np.random.default_rng(1)
    T, H, W, block = 4, 6, 10, (2, 3, 5)
    L = T * H * W
    x = rng.standard_normal((2, L, 3, 5))
    got = oracle.block_means(x, _members(T, H, W, block))
    # independent route: boolean mask from coordinates, then numpy's mean
    t, rem = np.divmod(np.arange(L), H * W)
    h, w = np.divmod(rem, W)
    bid = ((t // 2) * (H // 3) + h // 3) * (W // 5) + w // 5
    for i in range(got.shape[2]):
        ref = x[:, bid == i, :, :].mean(axis=1)
        np.testing.assert_allclose(got[:, :, i, :], ref, rtol=0, atol=1e-14)


def test_mean_of_block_means_is_global_mean():
    rng = np.random.default_rng(2)
    T, H, W = 6, 4, 8
    x = rng.standard_normal((1, T * H * W, 2, 4))
    for layer, block in [(0, (2, 4, 8)), (1, (6, 2, 2)), (2, (3, 2, 4))]:
        oracle.check_partition(T, H, W, layer, block)
        bm = oracle.block_means(x, _members(T, H, W, block))
        np.testing.assert_allclose(bm.mean(axis=2), x.mean(axis=1), atol=1e-14)


def test_linear_field_block_mean_is_value_at_block_centre():
    # closed form: the mean of an affine function over a box is its value at
    # the box centre
    T, H, W, block = 6, 8, 10, (3, 4, 5)
    a, b, c, e = 0.7, -1.3, 2.1, 0.4
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    x = (a * t + b * h + c * w + e).reshape(1, -1, 1, 1)
    bm = oracle.block_means(x, _members(T, H, W, block))[0, 0, :, 0]
    i = 0
    for it in range(T // 3):
        for ih in range(H // 4):
            for iw in range(W // 5):
                ct, ch, cw = it * 3 + 1.0, ih * 4 + 1.5, iw * 5 + 2.0
                assert bm[i] == pytest.approx(a * ct + b * ch + c * cw + e, abs=1e-12)
                i += 1
