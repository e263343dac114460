"""Pins for the oracle's dilation and groups functions.

Each check ties oracle.conv_general / conv_general_points / im2col_dilated /
out_dim_dilated to something other than themselves:
  * the output sizes the pages print (tests/golden/dilated_sizes.json, cited
    there, with the pages' wrong entries corrected by their own formula);
  * the plain oracle functions (pinned on their own in test_oracle_pins.py):
    d = 1, G = 1 reduces to them; a dilated kernel equals a plain kernel with
    zeros stuffed between its taps; G groups equal G plain convolutions of
    channel slices;
  * closed forms (depthwise on constant channels counts the in-range taps);
  * torch.nn.functional.conv2d / conv3d / unfold in float64 on the CPU;
  * brute force: per-group W_row @ X_col against the direct form.

A plausible mistake (dilation dropped from one axis, groups interleaved instead
of blocked, the group offset of the input channel lost, the dilated span
mis-sized, depth dilation lost, im2col ignoring dilation) fails at least one.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _rand(shape, rng, integer=False):
    if integer:
        return rng.integers(-2, 3, size=shape).astype(np.float32)
    return rng.standard_normal(size=shape).astype(np.float32)


# --- output size ---------------------------------------------------------------

def test_dilated_size_table(golden_dir):
    g = _load(golden_dir, "dilated_sizes.json")
    for c in g["cases"]:
        assert oracle.out_dim_dilated(c["in"], c["k"], c["s"], c["p"], c["d"]) == c["out"], c


def test_dilated_size_at_d1_is_plain_size(golden_dir):
    g = _load(golden_dir, "output_sizes.json")
    for c in g["cases"]:
        assert oracle.out_dim_dilated(c["in"], c["k"], c["s"], c["p"], 1) == c["out"], c


def test_dilated_size_rejects_bad_params():
    assert oracle.out_dim_dilated(9, 3, 1, 0, 0) == -1
    assert oracle.out_dim_dilated(9, 3, 0, 0, 2) == -1
    assert oracle.out_dim_dilated(4, 3, 1, 0, 2) == -1       # span 5 > 4
    assert oracle.out_dim_dilated(5, 1, 1, 0, 7) == 5        # one tap: dilation is moot


def test_dilated_size_brute_force():
    """Count window positions directly: the first tap at o*s - p, the last at
    o*s - p + d(K-1), both inside [-p, in + p)."""
    for n, k, s, p, d in itertools.product(range(1, 12), (1, 2, 3), (1, 2, 3), (0, 1, 2), (1, 2, 3)):
        cnt = 0
        while cnt * s + d * (k - 1) <= n + 2 * p - 1:
            cnt += 1
        assert oracle.out_dim_dilated(n, k, s, p, d) == (cnt if cnt else -1), (n, k, s, p, d)


# --- reductions to the plain oracle ---------------------------------------------

@pytest.mark.parametrize("ndim", [2, 3])
def test_d1_g1_equals_plain(ndim):
    rng = np.random.default_rng(5)
    if ndim == 2:
        x, w = _rand((2, 5, 7, 9), rng), _rand((6, 5, 3, 3), rng)
        ref, refS = oracle.conv2d(x, w, np.full((6,), 0.25, np.float32), 2, 1)
    else:
        x, w = _rand((2, 3, 5, 6, 7), rng), _rand((4, 3, 3, 3, 3), rng)
        ref, refS = oracle.conv3d(x, w, np.full((4,), 0.25, np.float32), 2, 1)
    y, S = oracle.conv_general(x, w, np.full((w.shape[0],), 0.25, np.float32), 2, 1, 1, 1)
    np.testing.assert_array_equal(y, ref)
    np.testing.assert_array_equal(S, refS)


def _stuff(w, d):
    """Plain kernel of size d(K-1)+1 with w's taps d apart and zeros between."""
    K = w.shape[2]
    Ke = d * (K - 1) + 1
    ws = np.zeros(w.shape[:2] + (Ke,) * (w.ndim - 2), w.dtype)
    ws[(slice(None), slice(None)) + (slice(None, None, d),) * (w.ndim - 2)] = w
    return ws


@pytest.mark.parametrize("H,W,K,s,p,d", [(9, 11, 3, 1, 2, 2), (12, 10, 3, 2, 1, 3), (8, 8, 2, 1, 0, 4),
                                          (7, 13, 5, 3, 4, 2)])
def test_dilation_equals_zero_stuffed_kernel_2d(H, W, K, s, p, d):
    rng = np.random.default_rng(H * 100 + d)
    x, w = _rand((2, 3, H, W), rng, True), _rand((4, 3, K, K), rng, True)
    b = _rand((4,), rng, True)
    y, _ = oracle.conv_general(x, w, b, s, p, d, 1)
    ref, _ = oracle.conv2d(x, _stuff(w, d), b, s, p)
    np.testing.assert_array_equal(y, ref)


def test_dilation_equals_zero_stuffed_kernel_3d():
    rng = np.random.default_rng(17)
    x, w = _rand((1, 2, 7, 8, 9), rng, True), _rand((3, 2, 3, 3, 3), rng, True)
    y, _ = oracle.conv_general(x, w, None, 1, 2, 2, 1)
    ref, _ = oracle.conv3d(x, _stuff(w, 2), None, 1, 2)
    np.testing.assert_array_equal(y, ref)


@pytest.mark.parametrize("ndim,C,Co,G,d", [(2, 8, 16, 4, 1), (2, 6, 9, 3, 2), (2, 4, 4, 4, 1),
                                           (2, 4, 8, 4, 3), (3, 6, 4, 2, 2), (3, 3, 6, 3, 1)])
def test_groups_are_independent_slices(ndim, C, Co, G, d):
    """Output block i is the plain convolution of input block i with the filters
    of block i [PyTorch tensor products and conv2d/conv3d dimension semantics,
    4.3; Conv2d from the official docs, 3.4]."""
    rng = np.random.default_rng(C * 7 + Co + G)
    sp = (9, 10) if ndim == 2 else (5, 6, 7)
    K, s, p = 3, 1, d
    x = _rand((2, C) + sp, rng, True)
    w = _rand((Co, C // G) + (K,) * ndim, rng, True)
    b = _rand((Co,), rng, True)
    y, S = oracle.conv_general(x, w, b, s, p, d, G)
    cg, og = C // G, Co // G
    plain = oracle.conv2d if ndim == 2 else oracle.conv3d
    for i in range(G):
        xs = x[:, i * cg:(i + 1) * cg].copy()
        ws = _stuff(w[i * og:(i + 1) * og], d).copy()
        ref, refS = plain(xs, ws, b[i * og:(i + 1) * og].copy(), s, p)
        np.testing.assert_array_equal(y[:, i * og:(i + 1) * og], ref)
        np.testing.assert_array_equal(S[:, i * og:(i + 1) * og], refS)


# --- closed forms -----------------------------------------------------------------

def _valid_taps_dil(o, s, p, K, d, n):
    return sum(1 for k in range(K) if 0 <= o * s + k * d - p < n)


@pytest.mark.parametrize("C,H,W,K,s,p,d,mult", [(5, 7, 9, 3, 1, 2, 2, 1), (4, 10, 6, 3, 2, 1, 3, 2),
                                                (3, 6, 6, 5, 1, 4, 2, 3)])
def test_depthwise_closed_form(C, H, W, K, s, p, d, mult):
    """Depthwise (G = C_in): input channel c holds the constant c+1 and all
    weights are 1, so output channel oc (group oc // mult) is (oc//mult + 1)
    times the number of in-range taps."""
    x = np.broadcast_to(np.arange(1, C + 1, dtype=np.float32)[None, :, None, None], (2, C, H, W)).copy()
    w = np.ones((C * mult, 1, K, K), np.float32)
    y, S = oracle.conv_general(x, w, None, s, p, d, C)
    Ho, Wo = y.shape[2:]
    assert (Ho, Wo) == (oracle.out_dim_dilated(H, K, s, p, d), oracle.out_dim_dilated(W, K, s, p, d))
    for oh, ow in itertools.product(range(Ho), range(Wo)):
        taps = _valid_taps_dil(oh, s, p, K, d, H) * _valid_taps_dil(ow, s, p, K, d, W)
        expect = (np.arange(C * mult) // mult + 1) * taps
        for n in range(2):
            np.testing.assert_array_equal(y[n, :, oh, ow], expect)
    np.testing.assert_array_equal(S, y)


def test_depthwise_example_shapes():
    """A 64-channel depthwise 3x3 layer has weight (64, 1, 3, 3): 64*9 weights
    and 64 biases, 640 parameters [PyTorch tensor products and conv2d/conv3d
    dimension semantics, 4.3]; a dense (64, 64, 3, 3) weight does not fit G = 64."""
    rng = np.random.default_rng(2)
    x = _rand((1, 64, 5, 5), rng)
    w = _rand((64, 1, 3, 3), rng)
    b = _rand((64,), rng)
    assert w.size + b.size == 640
    y, _ = oracle.conv_general(x, w, b, 1, 1, 1, 64)
    assert y.shape == (1, 64, 5, 5)
    # output channel c sees input channel c only
    for c in (0, 17, 63):
        ref, _ = oracle.conv2d(x[:, c:c + 1].copy(), w[c:c + 1].copy(), b[c:c + 1].copy(), 1, 1)
        np.testing.assert_array_equal(y[:, c:c + 1], ref)
    with pytest.raises(ValueError):
        oracle.conv_general(x, _rand((64, 64, 3, 3), rng), b, 1, 1, 1, 64)


def test_groups_example_8_to_16():
    """in 8, out 16, groups 4: weight (16, 2, 3, 3), four separate 2 -> 4
    convolutions [Conv2d from the official docs, 3.4].  Changing input group 0
    moves output channels 0..3 only."""
    rng = np.random.default_rng(3)
    x = _rand((2, 8, 6, 7), rng, True)
    w = _rand((16, 2, 3, 3), rng, True)
    y, _ = oracle.conv_general(x, w, None, 1, 1, 1, 4)
    x2 = x.copy()
    x2[:, 0:2] += 1.0
    y2, _ = oracle.conv_general(x2, w, None, 1, 1, 1, 4)
    changed = np.any(y2 != y, axis=(0, 2, 3))
    assert changed[:4].all() and not changed[4:].any()
    with pytest.raises(ValueError):
        oracle.conv_general(x, _rand((16, 8, 3, 3), rng), None, 1, 1, 1, 4)
    with pytest.raises(ValueError):
        oracle.conv_general(x, _rand((15, 2, 3, 3), rng), None, 1, 1, 1, 4)


# --- library special cases ----------------------------------------------------------

@pytest.mark.parametrize("N,C,H,W,Co,K,s,p,d,G", [
    (2, 8, 9, 11, 16, 3, 1, 1, 2, 4),
    (1, 6, 12, 10, 6, 3, 2, 2, 3, 6),       # depthwise, stride 2
    (2, 4, 7, 7, 8, 3, 1, 0, 2, 4),         # depthwise multiplier 2
    (1, 9, 8, 13, 6, 2, 3, 1, 2, 3),
    (3, 4, 16, 16, 4, 5, 1, 4, 2, 2),
])
def test_conv2d_general_matches_library(N, C, H, W, Co, K, s, p, d, G):
    rng = np.random.default_rng(N + C + H + d * 10 + G)
    x, w, b = _rand((N, C, H, W), rng), _rand((Co, C // G, K, K), rng), _rand((Co,), rng)
    y, _ = oracle.conv_general(x, w, b, s, p, d, G)
    ref = F.conv2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(), torch.from_numpy(b).double(),
                   stride=s, padding=p, dilation=d, groups=G).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N,C,D,H,W,Co,K,s,p,d,G", [
    (1, 4, 6, 7, 8, 6, 3, 1, 2, 2, 2),
    (2, 3, 5, 6, 7, 3, 3, 2, 1, 1, 3),
    (1, 2, 9, 8, 7, 4, 3, 1, 3, 3, 1),
])
def test_conv3d_general_matches_library(N, C, D, H, W, Co, K, s, p, d, G):
    rng = np.random.default_rng(N + C + D + d + G)
    x, w, b = _rand((N, C, D, H, W), rng), _rand((Co, C // G, K, K, K), rng), _rand((Co,), rng)
    y, _ = oracle.conv_general(x, w, b, s, p, d, G)
    ref = F.conv3d(torch.from_numpy(x).double(), torch.from_numpy(w).double(), torch.from_numpy(b).double(),
                   stride=s, padding=p, dilation=d, groups=G).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("K,s,p,d", [(3, 1, 2, 2), (3, 2, 1, 3), (2, 1, 0, 2), (1, 1, 0, 1)])
def test_im2col_dilated_matches_unfold(K, s, p, d):
    rng = np.random.default_rng(K * 10 + d)
    x = _rand((2, 3, 9, 10), rng)
    col = oracle.im2col_dilated(x, K, s, p, d)
    u = F.unfold(torch.from_numpy(x).double(), K, dilation=d, padding=p, stride=s)   # (N, C*K*K, L)
    ref = u.permute(1, 0, 2).reshape(u.shape[1], -1).numpy()
    np.testing.assert_array_equal(col, ref)


def test_im2col_dilated_at_d1_is_plain():
    rng = np.random.default_rng(4)
    x2, x3 = _rand((2, 3, 7, 8), rng), _rand((1, 2, 5, 6, 7), rng)
    np.testing.assert_array_equal(oracle.im2col_dilated(x2, 3, 2, 1, 1), oracle.im2col2d(x2, 3, 2, 1))
    np.testing.assert_array_equal(oracle.im2col_dilated(x3, 3, 1, 1, 1), oracle.im2col3d(x3, 3, 1, 1))


@pytest.mark.parametrize("ndim,C,Co,G,K,s,p,d", [(2, 8, 12, 4, 3, 1, 2, 2), (2, 6, 6, 6, 3, 2, 3, 3),
                                                 (3, 4, 6, 2, 3, 1, 2, 2), (3, 3, 3, 3, 2, 1, 1, 2)])
def test_grouped_im2col_gemm_equals_direct(ndim, C, Co, G, K, s, p, d):
    """Group i multiplies its filters' W_row (C_out/G x C_in/G * K^ndim) with
    its own row block of X_col [Why use matrix multiplication for convolution,
    2.3, applied per group]."""
    rng = np.random.default_rng(C + Co + G + d)
    sp = (8, 9) if ndim == 2 else (6, 5, 7)
    x = _rand((2, C) + sp, rng, True)
    w = _rand((Co, C // G) + (K,) * ndim, rng, True)
    col = oracle.im2col_dilated(x, K, s, p, d)
    y, _ = oracle.conv_general(x, w, None, s, p, d, G)
    N, plane = 2, int(np.prod(y.shape[2:]))
    rows, og = (C // G) * K ** ndim, Co // G
    for i in range(G):
        Y = oracle.matmul(w[i * og:(i + 1) * og].reshape(og, rows), col[i * rows:(i + 1) * rows])
        Y = Y.reshape(og, N, plane).transpose(1, 0, 2).reshape((N, og) + y.shape[2:])
        np.testing.assert_array_equal(Y, y[:, i * og:(i + 1) * og])


def test_general_S_is_conv_of_magnitudes():
    rng = np.random.default_rng(8)
    x, w = _rand((2, 6, 8, 9), rng), _rand((9, 2, 3, 3), rng)
    y, S = oracle.conv_general(x, w, None, 2, 2, 2, 3)
    yabs = oracle.conv_general(np.abs(x), np.abs(w), None, 2, 2, 2, 3, with_S=False)
    np.testing.assert_allclose(S, yabs, rtol=1e-14, atol=0)
    assert np.all(S >= np.abs(y) - 1e-12)


@pytest.mark.parametrize("ndim", [2, 3])
def test_general_points_match_full(ndim):
    rng = np.random.default_rng(9 + ndim)
    if ndim == 2:
        x, w = _rand((2, 8, 9, 10), rng), _rand((8, 2, 3, 3), rng)
    else:
        x, w = _rand((2, 4, 5, 6, 7), rng), _rand((8, 1, 3, 3, 3), rng)
    b = _rand((8,), rng)
    y, S = oracle.conv_general(x, w, b, 1, 2, 2, 4)
    idx = rng.choice(y.size, size=200, replace=False)
    yp, Sp = oracle.conv_general_points(x, w, b, 1, 2, 2, 4, idx)
    np.testing.assert_array_equal(yp, y.reshape(-1)[idx])
    np.testing.assert_array_equal(Sp, S.reshape(-1)[idx])
    with pytest.raises(ValueError):
        oracle.conv_general_points(x, w, b, 1, 2, 2, 4, np.array([y.size]))
