"""GPU parity for Winograd F(2x2, 3x3) (conv_fwd_ex_bf16 with
CONV_ALGO_WINOGRAD) against the oracle.

Acceptance is the same as every bf16 route: per output element
    |gpu - y_ref| <= 1e-3 * S,   S = sum |x w| of the direct convolution,
with y_ref and S from the direct fp64 oracle.  The bound the arithmetic
guarantees is looser: U and V are rounded to fp16 (unit roundoff 2^-11)
before the 16 products, so each product carries a relative error of at most
2^-10 (+2^-22), the fp32 sums over C_in add at most C_in * 2^-24 of the
magnitude and the output transform only adds and subtracts, which gives
|gpu - y_ref| <= 2^-9 * Sw with Sw the oracle's transform-domain magnitude sum
(about 1.7x, at most 4x, the direct S on N(0,1) data).  The tests assert the
contract bound and print the measured error against both.  On integer data
every transformed value is exact in fp16 (multiples of 1/4 up to 4.5 and
integers up to 8, times the power of two the route scales by) and every sum
exact in fp32, so the result must equal the direct convolution bit for bit.
The route scales x and w by powers of two chosen from their largest
magnitudes before rounding to fp16; inputs that fp16 could not hold
unscaled (|x| up to 2^22, or down at 2^-20) must meet the same contract.
"""
import numpy as np
import pytest
import torch

import oracle
from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import dev

pytestmark = pytest.mark.gpu
TAU = 1e-3          # the bf16 contract, relative to the direct S
TAU_W = 2.0 ** -9   # the derived transform-domain bound (diagnostic only)


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


def _check_contract(wl, t, got):
    """|gpu - y_ref| <= 1e-3 * S element by element (direct oracle); the
    transform-domain figure is printed beside it."""
    y_ref, S = oracle.conv2d(t.x, t.w, t.b, 1, wl.pad)
    assert got.shape == y_ref.shape
    d = np.abs(got - y_ref)
    bad = d > TAU * S
    _, Sw = oracle.winograd_f2x2_3x3(t.x, t.w, t.b, wl.pad)
    with np.errstate(divide="ignore", invalid="ignore"):
        rs = float(np.max(np.where(S > 0, d / np.where(S > 0, S, 1), 0.0)))
        rw = float(np.max(np.where(Sw > 0, d / np.where(Sw > 0, Sw, 1), 0.0)))
    print("winograd %s: max |d|/S = %.3g (contract %g), max |d|/Sw = %.3g (derived bound %.3g)" % (
        wl.x_shape, rs, TAU, rw, TAU_W))
    assert not bad.any(), "%d exceed 1e-3*S; first %s: gpu %r ref %r S %r" % (
        bad.sum(), tuple(np.argwhere(bad)[0]), got[bad][0], y_ref[bad][0], S[bad][0])


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
    _check_contract(wl, t, _run(wl, t))


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
    _check_contract(wl, t, _run(wl, t))


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


@pytest.mark.parametrize("xs,ws", [(2.0 ** 20, 2.0 ** 10), (2.0 ** -20, 2.0 ** -12), (3.0e4, 1.0), (1.0, 2.0 ** -30),
                                   (2.0 ** 60, 2.0 ** -70)],
                         ids=["huge", "tiny", "x_3e4", "w_2^-30", "x_2^60_w_2^-70"])
def test_winograd_magnitudes_outside_fp16(xs, ws):
    """x and w scaled far outside fp16's range (V would overflow to inf, or U
    and V sink into fp16 subnormals, without the route's own power-of-two
    scaling): the result still meets 1e-3 * S of the direct oracle."""
    wl = _wl(2, 64, 10, 16, 40, 1, seed=77)
    t = synth.make_inputs(wl)
    x = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(t.x) * np.float32(xs))
    w = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(t.w) * np.float32(ws))
    b = (t.b * np.float32(xs * ws)).astype(np.float32)
    t2 = synth.Tensors(x, w, b, t.seed)
    got = _run(wl, t2)
    assert np.isfinite(got).all()
    _check_contract(wl, t2, got)
