"""Pins of the oracle's index reordering (the 2-D-local flattening of the pages' Sec. 5.1 as read here:
recursive sqrt(B) x sqrt(B) tiles, so that every level-l unit is a square patch).

  * B = 4 with one top tile is the Morton (Z-order) curve: the position equals the bit interleave of (y, x);
  * every level-l unit (B^l consecutive tokens) is a sqrt(B)^l x sqrt(B)^l square of pixels, l <= L, also on
    non-square grids;
  * the map is a bijection, L = 0 is the identity, and moving rows there and back restores them;
  * a hand-worked 8 x 8 example (tests/golden/reorder_8x8_B16_L1.txt).
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "reorder_8x8_B16_L1.txt")


def _interleave(y, x, bits):
    z = 0
    for i in range(bits):
        z |= ((x >> i) & 1) << (2 * i)
        z |= ((y >> i) & 1) << (2 * i + 1)
    return z


@pytest.mark.parametrize("m", [1, 2, 3, 5])
def test_morton_for_block_4(m):
    H = W = 1 << m
    lo = oracle.reorder_index(H, W, 4, m).reshape(H, W)
    for y in range(H):
        for x in range(W):
            assert lo[y, x] == _interleave(y, x, m)


@pytest.mark.parametrize("H,W,B,L", [(64, 64, 16, 3), (64, 128, 16, 2), (48, 32, 16, 1), (32, 32, 4, 3),
                                     (27, 54, 9, 2)])
def test_units_are_square_patches(H, W, B, L):
    lo = oracle.reorder_index(H, W, B, L)
    assert np.array_equal(np.sort(lo), np.arange(H * W))  # bijection
    pos_y, pos_x = np.empty(H * W, np.int64), np.empty(H * W, np.int64)
    pos_y[lo] = np.repeat(np.arange(H), W)
    pos_x[lo] = np.tile(np.arange(W), H)
    s = int(round(B ** 0.5))
    for l in range(1, L + 1):
        side, size = s ** l, B ** l
        ys, xs = pos_y.reshape(-1, size), pos_x.reshape(-1, size)
        assert np.all(ys.max(1) - ys.min(1) == side - 1) and np.all(xs.max(1) - xs.min(1) == side - 1)
        assert np.all(ys.min(1) % side == 0) and np.all(xs.min(1) % side == 0)


def test_identity_and_round_trip():
    assert np.array_equal(oracle.reorder_index(16, 32, 16, 0), np.arange(16 * 32))
    lo = oracle.reorder_index(64, 64, 16, 2)
    x = np.random.default_rng(0).standard_normal((3, 64 * 64, 5))
    z = oracle.reorder(x, lo, True)
    assert np.array_equal(z[:, lo[77]], x[:, 77])
    assert np.array_equal(oracle.reorder(z, lo, False), x)


def test_golden_8x8():
    ref = np.loadtxt(GOLDEN, dtype=np.int64)
    assert np.array_equal(oracle.reorder_index(8, 8, 16, 1).reshape(8, 8), ref)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.reorder_index(8, 8, 8, 1)    # B not a square
    with pytest.raises(ValueError):
        oracle.reorder_index(24, 32, 16, 2)  # 16 does not divide 24
