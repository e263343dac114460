"""GPU parity for dilation and groups (including depthwise) against the
oracle's general convolution.

Every call goes through the general C entry points (conv_fwd_bf16,
conv_fwd_f32, conv_im2col_bf16, conv_fwd_explicit_bf16).  Routes: the
depthwise kernel (one input channel per group, 2D), the direct VALU kernel,
the MFMA implicit GEMM with one GEMM per group, and the explicit im2col +
per-group GEMM.  Sizes: small shapes spanning several tiles with ragged edges,
the three full-size layers (full-tensor comparison and integer-exact runs),
and degenerate cases (one tap in range, pad beyond the dilated span, a single
channel per group on both sides).
"""
import numpy as np
import pytest
import torch

import oracle
from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import TAU, compare, dev, poisoned, reference_general, run_general

pytestmark = pytest.mark.gpu

GENERAL_FULL = ["depthwise3x3_bf16", "dilated3x3_bf16", "grouped3x3_bf16"]


def _wl(name, ndim, N, C, sp, Co, K, s, p, d, g, dtype="bf16", dist="normal", seed=300):
    return synth.Workload(name, ndim, N, C, tuple(sp), Co, K, s, p, dtype, dist, seed, dilation=d, groups=g)


def _go(wl, t, route):
    if route == "explicit":
        return run_general(wl, t, explicit=True)
    return run_general(wl, t, algo=route)


# ---- grouped / dilated, every route ------------------------------------------

SMALL_GEN_2D = [
    # (N, C, H, W, Co, K, s, p, d, G)
    (2, 8, 13, 17, 16, 3, 1, 1, 1, 4),         # 2 -> 4 per group
    (2, 64, 12, 12, 64, 3, 1, 2, 2, 2),        # 32 -> 32 per group, dilated
    (1, 48, 9, 11, 96, 3, 2, 2, 3, 3),         # stride 2, dilation 3
    (3, 20, 10, 14, 70, 3, 1, 1, 2, 1),        # dilation only, ragged channels
    (1, 128, 8, 8, 256, 3, 1, 1, 1, 2),        # wide groups: several MFMA row tiles
    (2, 12, 15, 9, 12, 5, 1, 4, 2, 6),         # 2 -> 2 per group, K 5
    (1, 6, 5, 5, 6, 3, 1, 3, 3, 1),            # only the centre tap lands for most outputs
    (1, 4, 3, 3, 8, 3, 1, 5, 2, 2),            # pad beyond the dilated span: bias-only borders
]


@pytest.mark.parametrize("shape", SMALL_GEN_2D, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("route", ["auto", "mfma", "valu", "explicit"])
def test_small_general_2d(shape, route):
    N, C, H, W, Co, K, s, p, d, g = shape
    wl = _wl("gen2d", 2, N, C, (H, W), Co, K, s, p, d, g)
    t = synth.make_inputs(wl, seed=sum(shape))
    y_ref, S = reference_general(wl, t)
    compare(_go(wl, t, route), y_ref, S, TAU["bf16"], label="%s %s" % (shape, route))


SMALL_GEN_3D = [
    # (N, C, D, H, W, Co, K, s, p, d, G)
    (2, 4, 6, 7, 8, 6, 3, 1, 2, 2, 2),
    (1, 6, 5, 6, 7, 9, 3, 2, 1, 1, 3),
    (1, 32, 4, 6, 6, 64, 3, 1, 2, 2, 2),
    (1, 3, 7, 6, 5, 3, 3, 1, 1, 2, 3),        # depthwise 3D: direct VALU / MFMA
]


@pytest.mark.parametrize("shape", SMALL_GEN_3D, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("route", ["auto", "mfma", "valu", "explicit"])
def test_small_general_3d(shape, route):
    N, C, D, H, W, Co, K, s, p, d, g = shape
    wl = _wl("gen3d", 3, N, C, (D, H, W), Co, K, s, p, d, g, dist="uniform")
    t = synth.make_inputs(wl, seed=sum(shape))
    y_ref, S = reference_general(wl, t)
    compare(_go(wl, t, route), y_ref, S, TAU["bf16"], label="%s %s" % (shape, route))


# ---- depthwise kernel ----------------------------------------------------------

DEPTHWISE = [
    # (N, C, H, W, mult, K, s, p, d)
    (2, 8, 20, 40, 1, 3, 1, 1, 1),             # two column tiles (64 wide), ragged
    (1, 5, 33, 70, 1, 3, 1, 1, 1),             # rows over several 16-row tiles
    (2, 6, 17, 19, 2, 3, 2, 1, 1),             # multiplier 2, stride 2, 32-wide tiles
    (1, 4, 30, 30, 3, 5, 1, 4, 2),             # K 5, dilation 2, multiplier 3
    (1, 3, 12, 100, 1, 3, 2, 3, 3),            # stride 2 + dilation 3
    (2, 16, 7, 7, 1, 7, 1, 3, 1),              # K 7 (runtime K)
    (1, 2, 1, 1, 4, 3, 1, 1, 1),               # 1x1 input: only the centre tap
    (1, 1, 9, 9, 8, 3, 1, 1, 1),               # C_in = 1, groups = 1: one channel, 8 filters
    (1, 4097, 32, 32, 1, 3, 1, 1, 1),          # 4097 tiles: two tiles per workgroup, odd tail
    (1, 16387, 8, 16, 1, 3, 2, 1, 1),          # 16387 tiles: eight per workgroup, ragged tail
]


@pytest.mark.parametrize("shape", DEPTHWISE, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("with_bias", [True, False])
def test_depthwise_kernel(shape, dtype, with_bias):
    N, C, H, W, mult, K, s, p, d = shape
    wl = _wl("dw", 2, N, C, (H, W), C * mult, K, s, p, d, C, dtype=dtype)
    t = synth.make_inputs(wl, seed=sum(shape) + 7, with_bias=with_bias)
    y_ref, S = reference_general(wl, t)
    compare(_go(wl, t, "valu"), y_ref, S, TAU[dtype], label="%s %s" % (shape, dtype))


@pytest.mark.parametrize("shape", DEPTHWISE[:4], ids=lambda s: "x".join(map(str, s)))
def test_depthwise_integer_exact(shape):
    N, C, H, W, mult, K, s, p, d = shape
    wl = _wl("dw", 2, N, C, (H, W), C * mult, K, s, p, d, C)
    t = synth.make_inputs(wl, seed=11, integer=True)
    y_ref, S = reference_general(wl, t)
    compare(_go(wl, t, "auto"), y_ref, S, 0, exact=True, label=str(shape))


def test_general_f32_direct():
    for shape in [(2, 6, 9, 11, 9, 3, 2, 2, 2, 3), (1, 8, 7, 7, 4, 3, 1, 2, 2, 2)]:
        N, C, H, W, Co, K, s, p, d, g = shape
        wl = _wl("genf32", 2, N, C, (H, W), Co, K, s, p, d, g, dtype="f32", dist="uniform")
        t = synth.make_inputs(wl, seed=sum(shape))
        y_ref, S = reference_general(wl, t)
        compare(_go(wl, t, "valu"), y_ref, S, TAU["f32"], label=str(shape))


# ---- dilation 2 on the column-group kernel (workspace entry point) ---------------

DILATED_CG = [
    # (N, C, H, W, C_out): K 3, stride 1, pad 2, dilation 2
    (2, 32, 19, 40, 128),      # two bands of 16 rows, the last one ragged; both row phases
    (1, 16, 5, 32, 128),       # one 16-channel stage, fewer rows than a tile, W = 32
    (1, 48, 33, 64, 256),      # W = 64 (the widest tile), two 128-channel blocks
    (2, 64, 12, 48, 128),
]


@pytest.mark.parametrize("shape", DILATED_CG, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("integer", [False, True])
def test_dilated_column_group(shape, integer):
    N, C, H, W, Co = shape
    wl = _wl("dilcg", 2, N, C, (H, W), Co, 3, 1, 2, 2, 1)
    t = synth.make_inputs(wl, seed=sum(shape), integer=integer)
    y_ref, S = reference_general(wl, t)
    ws = B.workspace_ex(wl.x_shape, wl.w_shape, 1, 2, 2, 1, "nchw", "f32", False, "auto")
    assert ws is not None and ws.numel() == Co * C * 9 * 2     # packed weights: the column-group route
    y = B.conv_ex(dev(t.x, None), dev(t.w, None), dev(t.b, np.float32), 1, 2, 2, 1, "nchw", "f32", False, "auto",
                  ws, out=poisoned(wl.y_shape))
    torch.cuda.synchronize()
    compare(y.cpu().numpy(), y_ref, S, 0 if integer else TAU["bf16"], exact=integer, label=str(shape))


# ---- groups of 32 output channels on the column-group kernel (workspace entry point)

GROUPED_CG = [
    # (N, C, H, W, C_out, G): K 3, stride 1, pad 1; C_out / G = 32
    (2, 128, 19, 40, 128, 4),    # two input stages per group, ragged last row tile
    (1, 64, 9, 56, 128, 4),      # 16 input channels per group: one stage; two loader passes (W = 56)
    (1, 256, 10, 32, 256, 8),    # two 128-channel blocks, W = 32
    (2, 128, 8, 48, 128, 4),
]


@pytest.mark.parametrize("shape", GROUPED_CG, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("integer", [False, True])
def test_grouped_column_group(shape, integer):
    N, C, H, W, Co, g = shape
    wl = _wl("grpcg", 2, N, C, (H, W), Co, 3, 1, 1, 1, g)
    t = synth.make_inputs(wl, seed=sum(shape), integer=integer)
    y_ref, S = reference_general(wl, t)
    ws = B.workspace_ex(wl.x_shape, wl.w_shape, 1, 1, 1, g, "nchw", "f32", False, "auto")
    assert ws is not None and ws.numel() == Co * (C // g) * 9 * 2     # packed weights: the column-group route
    y = B.conv_ex(dev(t.x, None), dev(t.w, None), dev(t.b, np.float32), 1, 1, 1, g, "nchw", "f32", False, "auto",
                  ws, out=poisoned(wl.y_shape))
    torch.cuda.synchronize()
    compare(y.cpu().numpy(), y_ref, S, 0 if integer else TAU["bf16"], exact=integer, label=str(shape))


@pytest.mark.parametrize("integer", [False, True])
def test_grouped_full_layer_column_group(integer):
    """The G = 4 layer (64,128,56,56) through the workspace entry point, whole output."""
    wl = synth.ALL_WORKLOADS["grouped3x3_bf16"]
    t = synth.make_inputs(wl, integer=integer)
    y_ref, S = reference_general(wl, t)
    ws = B.workspace_ex(wl.x_shape, wl.w_shape, 1, 1, 1, wl.groups, "nchw", "f32", False, "auto")
    assert ws is not None and ws.numel() == 128 * 32 * 9 * 2
    y = B.conv_ex(dev(t.x, None), dev(t.w, None), dev(t.b, np.float32), 1, 1, 1, wl.groups, "nchw", "f32", False,
                  "auto", ws, out=poisoned(wl.y_shape))
    torch.cuda.synchronize()
    compare(y.cpu().numpy(), y_ref, S, 0 if integer else TAU["bf16"], exact=integer, label="grouped full")


# ---- full-size layers ----------------------------------------------------------

@pytest.mark.parametrize("name", GENERAL_FULL)
def test_general_full_workload(name):
    wl = synth.ALL_WORKLOADS[name]
    t = synth.make_inputs(wl)
    y_ref, S = reference_general(wl, t)
    compare(_go(wl, t, "auto"), y_ref, S, TAU["bf16"], label=name)


@pytest.mark.parametrize("name", GENERAL_FULL)
def test_general_full_workload_integer_exact(name):
    wl = synth.ALL_WORKLOADS[name]
    t = synth.make_inputs(wl, integer=True)
    y_ref, S = reference_general(wl, t)
    compare(_go(wl, t, "auto"), y_ref, S, 0, exact=True, label=name)


@pytest.mark.parametrize("name", ["dilated3x3_bf16", "grouped3x3_bf16"])
@pytest.mark.parametrize("route", ["valu", "explicit"])
def test_general_full_other_routes_sampled(name, route):
    """The other routes at full size, checked on sampled outputs."""
    wl = synth.ALL_WORKLOADS[name]
    t = synth.make_inputs(wl)
    y = _go(wl, t, route)
    rng = np.random.default_rng(5)
    idx = rng.choice(y.size, size=4000, replace=False)
    y_ref, S = oracle.conv_general_points(t.x, t.w, t.b, wl.stride, wl.pad, wl.dilation, wl.groups, idx)
    compare(y.reshape(-1)[idx], y_ref, S, TAU["bf16"], label="%s %s" % (name, route))


# ---- d = 1, G = 1 is the plain problem -------------------------------------------

@pytest.mark.parametrize("name", ["stem_bf16", "conv1x1_bf16", "conv3d_bf16"])
def test_general_entry_matches_plain_entry(name):
    wl = synth.WORKLOADS[name]
    t = synth.make_inputs(wl)
    x, w, b = dev(t.x, np.float32), dev(t.w, np.float32), dev(t.b, np.float32)
    y1 = B.conv(x, w, b, wl.stride, wl.pad)
    y2 = B.conv_general(x, w, b, wl.stride, wl.pad, 1, 1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ---- dilated im2col ----------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2, 3, 9, 11, 3, 1, 2, 2), (1, 5, 12, 10, 3, 2, 3, 3), (2, 4, 8, 8, 2, 1, 1, 4),
                                   (2, 4, 8, 16, 3, 1, 2, 2), (1, 3, 6, 24, 3, 1, 3, 3)])
def test_im2col_dilated_bit_exact(shape):
    N, C, H, W, K, s, p, d = shape
    wl = _wl("col", 2, N, C, (H, W), 1, K, s, p, d, 1)
    t = synth.make_inputs(wl, seed=sum(shape))
    col = B.im2col_general(dev(t.x, np.float32), K, s, p, d)
    torch.cuda.synchronize()
    got = synth.bf16_bits_to_f32(col.cpu().numpy().view(np.uint16)).astype(np.float64)
    np.testing.assert_array_equal(got, oracle.im2col_dilated(t.x, K, s, p, d))


def test_im2col_dilated_3d_bit_exact():
    wl = _wl("col3", 3, 1, 2, (6, 7, 8), 1, 3, 1, 2, 2, 1, dist="uniform")
    t = synth.make_inputs(wl, seed=3)
    col = B.im2col_general(dev(t.x, np.float32), 3, 1, 2, 2)
    torch.cuda.synchronize()
    got = synth.bf16_bits_to_f32(col.cpu().numpy().view(np.uint16)).astype(np.float64)
    np.testing.assert_array_equal(got, oracle.im2col_dilated(t.x, 3, 1, 2, 2))


def test_general_validation_leaves_output_untouched():
    wl = _wl("v", 2, 1, 8, (9, 9), 8, 3, 1, 1, 1, 4)
    t = synth.make_inputs(wl, seed=1)
    x, w = dev(t.x, np.float32), dev(t.w, np.float32)
    y = poisoned(wl.y_shape)
    prm = B.make_params(tuple(x.shape), tuple(w.shape), 1, 1, 1, 3)       # groups 3 does not divide 8
    assert B.conv_fwd_bf16(prm, x.data_ptr(), w.data_ptr(), None, y.data_ptr(), 0, None) == 2
    torch.cuda.synchronize()
    assert torch.isnan(y).all()
