"""Pins for the oracle's output epilogue (ReLU, bf16 rounding) and its
channels-last convolution.

  * bf16 rounding against torch's float32 -> bfloat16 conversion (round to
    nearest even) on random and hand-picked values, ties included, and
    against its definition (the result has an 8-bit significand and is the
    nearest such value);
  * ReLU against its definition on signed data;
  * the channels-last convolution against the NCHW oracle (pinned elsewhere)
    through numpy transposes, and against torch on channels-last tensors.

A plausible mistake (ties rounded away from zero, truncation, ReLU keeping
negatives, the channel offset of a group lost in the channels-last index)
fails at least one.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _torch_bf16(a):
    return torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch_random():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        rng.integers(-70000, 70000, 5000)]).astype(np.float32)
    got = np.array([oracle.round_bf16(float(a)) for a in v])
    np.testing.assert_array_equal(got, _torch_bf16(v))
    np.testing.assert_array_equal(oracle.epilogue(v.astype(np.float64), to_bf16=True), got)


@pytest.mark.parametrize("v,expect", [
    (1.0 + 2.0 ** -8, 1.0),                    # tie: even significand below
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),    # tie: even significand above
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -7),
    (-(1.0 + 2.0 ** -8), -1.0),
    (257.0, 256.0), (259.0, 260.0), (255.0, 255.0),
    (0.0, 0.0), (-0.0, -0.0),
])
def test_round_bf16_ties_and_exact_integers(v, expect):
    assert oracle.round_bf16(v) == expect
    assert _torch_bf16([v])[0] == expect


def test_round_bf16_is_nearest_8_bit_significand():
    rng = np.random.default_rng(1)
    for v in rng.standard_normal(300) * 1e3:
        r = oracle.round_bf16(v)
        m, e = np.frexp(r)
        assert m * 256 == np.round(m * 256)                 # 8 significant bits
        ulp = 2.0 ** (np.frexp(v)[1] - 8)
        assert abs(r - v) <= ulp / 2


def test_relu_and_order():
    """ReLU first, then rounding: on fp32-representable values the result is
    torch's bf16 of max(y, 0)."""
    rng = np.random.default_rng(2)
    y = (rng.standard_normal(1000) * 5).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(oracle.epilogue(y, relu=True), np.maximum(y, 0.0))
    np.testing.assert_array_equal(oracle.epilogue(y), y)
    both = oracle.epilogue(y, relu=True, to_bf16=True)
    np.testing.assert_array_equal(both, _torch_bf16(np.maximum(y, 0.0)))
    assert np.all(both >= 0) and np.any(y < 0)


@pytest.mark.parametrize("ndim,N,C,sp,Co,K,s,p,d,G", [
    (2, 2, 6, (7, 9), 8, 3, 1, 1, 1, 1),
    (2, 1, 8, (9, 8), 12, 3, 2, 2, 2, 4),
    (2, 2, 4, (6, 6), 4, 3, 1, 1, 1, 4),      # depthwise
    (3, 1, 4, (5, 6, 7), 6, 3, 1, 1, 1, 2),
])
def test_nhwc_equals_nchw(ndim, N, C, sp, Co, K, s, p, d, G):
    rng = np.random.default_rng(C + Co)
    x = rng.integers(-2, 3, size=(N, C) + sp).astype(np.float64)
    w = rng.integers(-2, 3, size=(Co, C // G) + (K,) * ndim).astype(np.float64)
    b = rng.integers(-3, 4, size=Co).astype(np.float64)
    y, S = oracle.conv_general(x, w, b, s, p, d, G)
    to_last = (0,) + tuple(range(2, ndim + 2)) + (1,)
    yl, Sl = oracle.conv_nhwc(np.ascontiguousarray(x.transpose(to_last)), w, b, s, p, d, G)
    np.testing.assert_array_equal(yl, y.transpose(to_last))
    np.testing.assert_array_equal(Sl, S.transpose(to_last))


def test_nhwc_matches_library_channels_last():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 16, 9, 11))
    w = rng.standard_normal((32, 8, 3, 3))
    xt = torch.tensor(x).to(memory_format=torch.channels_last)
    ref = F.conv2d(xt, torch.tensor(w), stride=2, padding=1, groups=2)
    yl = oracle.conv_nhwc(np.ascontiguousarray(x.transpose(0, 2, 3, 1)), w, None, 2, 1, 1, 2, with_S=False)
    np.testing.assert_allclose(yl, ref.permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)
