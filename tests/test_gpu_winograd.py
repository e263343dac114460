"""GPU parity for Winograd F(2x2, 3x3) (conv_fwd_ex_bf16 with
CONV_ALGO_WINOGRAD) against the oracle's Winograd (which equals the direct
convolution in fp64).

Tolerance, derived from the arithmetic: the transformed filter U and input
block V are rounded to fp16 (unit roundoff 2^-11) before the 16 products, so
each product carries a relative error of at most 2^-10 (+2^-22), the fp32 sums
over C_in add at most C_in * 2^-24 of the magnitude, and the output transform
only adds and subtracts.  Per output
    |gpu - y_ref| <= 2^-9 * Sw,
Sw being the oracle's transform-domain magnitude sum (sum over channels and
points of |A coeff| |U| |V|), which is about 1.7x (up to 4x) the direct
S = sum |x w| on N(0,1) data.  On integer data every transformed value is
exact in fp16 (multiples of 1/4 up to 4.5 and integers up to 8) and every sum
exact in fp32, so the result must equal the direct convolution bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import dev

pytestmark = pytest.mark.gpu
TAU_W = 2.0 ** -9


def _wl(N, C, H, W, Co, p, seed=700):
    return synth.Workload("wino", 2, N, C, (H, W), Co, 3, 1, p, "bf16", "normal", seed)


def _run(wl, t, out_dtype="f32", relu=False):
    x, w, b = dev(t.x, None), dev(t.w, None), dev(t.b, np.float32)
    ws = B.workspace_ex(wl.x_shape, wl.w_shape, 1, wl.pad, algo="winograd", out_dtype=out_dtype, relu=relu)
    assert ws is not None
    y = B.conv_ex(x, w, b, 1, wl.pad, out_dtype=out_dtype, relu=relu, algo="winograd", workspace=ws)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    if out_dtype == "bf16":
        y = synth.bf16_bits_to_f32(y.view(np.uint16))
    return y.astype(np.float64)


SHAPES = [
    (2, 16, 9, 11, 24, 1),       # odd output: cropped last block row and column
    (1, 32, 8, 8, 64, 0),        # pad 0
    (2, 16, 7, 13, 130, 2),      # C_out past four 32-row tiles, pad 2
    (3, 48, 12, 10, 40, 1),      # several block tiles of 32
    (1, 16, 1, 1, 8, 1),         # one input pixel: only the centre tap
    # C_in % 32 == 0 and W % 8 == 0: the input transform from LDS tiles of 32 channels x 32 blocks
    (2, 64, 10, 16, 40, 1),      # pad 1: the tile starts one pixel left of the image
    (1, 32, 9, 40, 16, 2),       # pad 2, odd height
    (2, 96, 6, 72, 32, 1),       # 37 blocks a row: a second, ragged block tile
    (1, 32, 16, 8, 8, 3),        # pad 3
    (1, 64, 5, 64, 24, 0),       # pad 0, 31 blocks a row
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_winograd_small(shape):
    wl = _wl(*shape)
    t = synth.make_inputs(wl, seed=sum(shape))
    y_ref, Sw = oracle.winograd_f2x2_3x3(t.x, t.w, t.b, wl.pad)
    got = _run(wl, t)
    assert got.shape == y_ref.shape
    d = np.abs(got - y_ref)
    bad = d > TAU_W * Sw
    assert not bad.any(), "%d exceed; first %s: gpu %r ref %r Sw %r" % (
        bad.sum(), tuple(np.argwhere(bad)[0]), got[bad][0], y_ref[bad][0], Sw[bad][0])


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_winograd_integer_exact(shape):
    wl = _wl(*shape)
    t = synth.make_inputs(wl, seed=5, integer=True)
    y_ref, _ = oracle.conv2d(t.x, t.w, t.b, 1, wl.pad)
    got = _run(wl, t)
    np.testing.assert_array_equal(got, y_ref)


def test_winograd_epilogue_bf16_relu_integer_exact():
    wl = _wl(2, 16, 9, 11, 24, 1)
    t = synth.make_inputs(wl, seed=6, integer=True)
    y_ref, _ = oracle.conv2d(t.x, t.w, t.b, 1, 1)
    got = _run(wl, t, "bf16", True)
    np.testing.assert_array_equal(got, oracle.epilogue(y_ref, relu=True, to_bf16=True))


def test_winograd_full_3x3_layer():
    wl = synth.WORKLOADS["conv3x3_bf16"]
    t = synth.make_inputs(wl)
    y_ref, Sw = oracle.winograd_f2x2_3x3(t.x, t.w, t.b, 1)
    got = _run(wl, t)
    d = np.abs(got - y_ref)
    assert np.all(d <= TAU_W * Sw), float(np.max(d / np.maximum(Sw, 1e-30)))


def test_winograd_validation():
    wl = _wl(1, 16, 8, 8, 16, 1)
    t = synth.make_inputs(wl, seed=1)
    x, w = dev(t.x, None), dev(t.w, None)
    y = torch.full(wl.y_shape, float("nan"), device="cuda")
    prm = B.make_params(wl.x_shape, wl.w_shape, 1, 1)
    # no workspace
    assert B.conv_fwd_ex_bf16(prm, None, x.data_ptr(), w.data_ptr(), None, y.data_ptr(), None, 0, 3, None) == 6
    # 5x5 or C_in % 16 != 0: not a Winograd shape
    prm5 = B.make_params((1, 16, 8, 8), (16, 16, 5, 5), 1, 2)
    assert B.conv_fwd_ex_workspace_bytes(prm5, None, 3) == 0
    assert B.conv_fwd_ex_bf16(prm5, None, x.data_ptr(), w.data_ptr(), None, y.data_ptr(), None, 0, 3, None) == 7
    # the plain entry points do not take Winograd
    assert B.conv2d_fwd_bf16(x.data_ptr(), w.data_ptr(), None, y.data_ptr(), 1, 16, 8, 8, 16, 3, 1, 1, 3, None) == 7
    torch.cuda.synchronize()
    assert torch.isnan(y).all()
