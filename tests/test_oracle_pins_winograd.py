"""Pins for the oracle's Winograd F(2x2, 3x3) (oracle.winograd_f2x2_3x3).

  * on integer data it equals the direct convolution oracle (pinned elsewhere)
    exactly -- every transform coefficient is 0, +-1 or +-1/2 -- for pads 0-2,
    odd and even output sizes (cropped last blocks), one and many channels;
  * on random data it agrees to fp64 rounding (1e-12 of the direct S);
  * a hand-computed case: a 4x4 ramp under an all-ones 3x3 filter, pad 0,
    gives the 2x2 block [[45, 54], [81, 90]];
  * its magnitude sum bounds the result: Sw >= |y - bias|.

A plausible mistake (a sign in B^T, a coefficient of G, a row of A^T, the
crop of the last block) fails at least one.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("N,C,H,W,Co,p", [(2, 5, 9, 11, 4, 1), (1, 1, 4, 4, 1, 0), (1, 3, 7, 8, 2, 2),
                                          (2, 16, 12, 10, 8, 1), (1, 2, 5, 6, 3, 0), (1, 4, 1, 1, 2, 1)])
def test_winograd_equals_direct_on_integers(N, C, H, W, Co, p):
    rng = np.random.default_rng(N + C + H + W + p)
    x = rng.integers(-3, 4, (N, C, H, W)).astype(np.float64)
    w = rng.integers(-3, 4, (Co, C, 3, 3)).astype(np.float64)
    b = rng.integers(-3, 4, Co).astype(np.float64)
    y, Sw = oracle.winograd_f2x2_3x3(x, w, b, p)
    yd, _ = oracle.conv2d(x, w, b, 1, p)
    np.testing.assert_array_equal(y, yd)
    assert np.all(Sw >= np.abs(y - b[None, :, None, None]))


def test_winograd_random_data():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 8, 13, 10))
    w = rng.standard_normal((6, 8, 3, 3))
    y, _ = oracle.winograd_f2x2_3x3(x, w, None, 1)
    yd, S = oracle.conv2d(x, w, None, 1, 1)
    assert np.all(np.abs(y - yd) <= 1e-12 * S)


def test_winograd_hand_case():
    x = np.arange(16, dtype=np.float64).reshape(1, 1, 4, 4)
    w = np.ones((1, 1, 3, 3))
    y, Sw = oracle.winograd_f2x2_3x3(x, w, None, 0)
    np.testing.assert_array_equal(y[0, 0], [[45.0, 54.0], [81.0, 90.0]])


def test_winograd_rejects_other_kernels():
    with pytest.raises(ValueError):
        oracle.winograd_f2x2_3x3(np.zeros((1, 2, 5, 5)), np.zeros((1, 2, 5, 5)), None, 1)
