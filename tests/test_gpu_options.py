"""GPU parity for the forward options: channels-last layout, ReLU, bf16 output
(conv_fwd_ex_bf16 / conv_fwd_ex_f32) against the oracle's convolution (NCHW or
channels-last) followed by its epilogue.

Acceptance per element, in fp64: with ref = relu?(y_oracle),
  fp32 output:  |gpu - ref| <= tau * S
  bf16 output:  |gpu - ref| <= tau * S + 2^-8 * |ref|
(rounding an fp32 result to bf16 moves it by at most 2^-9 of its magnitude;
the bound leaves room for the fp32 error).  Integer-valued inputs keep every
fp32 result exact, so there the output must equal the oracle's epilogue
(ReLU, then round to nearest even) bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import TAU, dev

pytestmark = pytest.mark.gpu


def _wl(ndim, N, C, sp, Co, K, s, p, d, G, dtype="bf16", seed=500):
    return synth.Workload("opt", ndim, N, C, tuple(sp), Co, K, s, p, dtype, "normal", seed, dilation=d, groups=G)


def _to_last(a, ndim):
    return np.ascontiguousarray(a.transpose((0,) + tuple(range(2, ndim + 2)) + (1,)))


def _run(wl, t, layout, out_dtype, relu, algo, use_ws=False):
    x = t.x if layout == "nchw" else _to_last(t.x, wl.ndim)
    xt = dev(x, np.float32)
    wt, bt = dev(t.w, np.float32), dev(t.b, np.float32)
    ws = None
    if use_ws:
        ws = B.workspace_ex(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups, layout, out_dtype,
                            relu, algo)
    y = B.conv_ex(xt, wt, bt, wl.stride, wl.pad, wl.dilation, wl.groups, layout, out_dtype, relu, algo, ws)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    if out_dtype == "bf16":
        y = synth.bf16_bits_to_f32(y.view(np.uint16))
    return y.astype(np.float64)


def _reference(wl, t, layout):
    if layout == "nchw":
        return oracle.conv_general(t.x, t.w, t.b, wl.stride, wl.pad, wl.dilation, wl.groups)
    return oracle.conv_nhwc(_to_last(t.x, wl.ndim), t.w, t.b, wl.stride, wl.pad, wl.dilation, wl.groups)


def _check(got, y_ref, S, relu, out_dtype, tau, exact, label):
    assert got.shape == y_ref.shape, (label, got.shape, y_ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % label
    if exact:
        want = oracle.epilogue(y_ref, relu=relu, to_bf16=out_dtype == "bf16")
        bad = got != want
        assert not bad.any(), "%s: %d differ; first at %s gpu %r want %r" % (
            label, bad.sum(), tuple(np.argwhere(bad)[0]), got[bad][0], want[bad][0])
        return
    ref = oracle.epilogue(y_ref, relu=relu)
    bound = tau * S + (2.0 ** -8 * np.abs(ref) if out_dtype == "bf16" else 0.0)
    d = np.abs(got - ref)
    bad = d > bound
    assert not bad.any(), "%s: %d exceed the bound; first at %s gpu %r ref %r S %r" % (
        label, bad.sum(), tuple(np.argwhere(bad)[0]), got[bad][0], ref[bad][0], S[bad][0])


CASES = [
    # (name, (ndim, N, C, sp, Co, K, s, p, d, G), algo, use_ws)
    ("3x3 column-group", (2, 2, 128, (56, 56), 128, 3, 1, 1, 1, 1), "auto", True),
    ("3x3 W=40 column-group", (2, 1, 32, (13, 40), 256, 3, 1, 1, 1, 1), "auto", True),
    ("3x3 dilation 2 column-group", (2, 2, 32, (19, 40), 128, 3, 1, 2, 2, 1), "auto", True),
    ("3x3 groups of 32 column-group", (2, 2, 128, (11, 40), 128, 3, 1, 1, 1, 4), "auto", True),
    ("pointwise", (2, 3, 64, (14, 16), 192, 1, 1, 0, 1, 1), "auto", False),
    ("depthwise", (2, 2, 24, (30, 40), 48, 3, 2, 1, 1, 24), "auto", False),
    ("stem (short-reduction kernel)", (2, 2, 3, (33, 35), 64, 3, 2, 1, 1, 1), "auto", False),
    ("general MFMA, groups + dilation", (2, 2, 48, (17, 19), 96, 3, 1, 2, 2, 3), "mfma", False),
    ("general VALU", (2, 2, 6, (11, 9), 10, 3, 2, 1, 1, 2), "valu", False),
    ("3D general", (3, 1, 16, (5, 9, 10), 40, 3, 1, 1, 1, 1), "mfma", False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("opts", [("nchw", "bf16", False), ("nchw", "f32", True), ("nchw", "bf16", True),
                                  ("nhwc", "f32", False), ("nhwc", "bf16", True)],
                         ids=lambda o: "-".join(str(v) for v in o))
def test_options(case, opts):
    name, shape, algo, use_ws = case
    layout, out_dtype, relu = opts
    wl = _wl(*shape)
    t = synth.make_inputs(wl, seed=sum(shape[3]) + shape[4])
    y_ref, S = _reference(wl, t, layout)
    got = _run(wl, t, layout, out_dtype, relu, algo, use_ws)
    _check(got, y_ref, S, relu, out_dtype, TAU["bf16"], False, "%s %s" % (name, opts))


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
def test_options_integer_exact(case, layout):
    name, shape, algo, use_ws = case
    wl = _wl(*shape)
    t = synth.make_inputs(wl, seed=3, integer=True)
    y_ref, _ = _reference(wl, t, layout)
    got = _run(wl, t, layout, "bf16", True, algo, use_ws)
    _check(got, y_ref, None, True, "bf16", 0, True, "%s %s" % (name, layout))


def test_f32_inputs_channels_last():
    wl = _wl(2, 2, 5, (9, 11), 7, 3, 2, 1, 1, 1, dtype="f32")
    t = synth.make_inputs(wl, seed=9)
    y_ref, S = _reference(wl, t, "nhwc")
    got = _run(wl, t, "nhwc", "f32", True, "auto")
    _check(got, y_ref, S, True, "f32", TAU["f32"], False, "fp32 nhwc relu")


def test_full_3x3_layer_bf16_relu():
    """The 3x3 layer (64,128,56,56) with the bf16 + ReLU epilogue on the column-group kernel."""
    wl = synth.WORKLOADS["conv3x3_bf16"]
    t = synth.make_inputs(wl)
    y_ref, S = _reference(wl, t, "nchw")
    got = _run(wl, t, "nchw", "bf16", True, "auto", True)
    _check(got, y_ref, S, True, "bf16", TAU["bf16"], False, "full 3x3 bf16 relu")


@pytest.mark.parametrize("layout,out_dtype,relu", [("nhwc", "f32", False), ("nhwc", "bf16", True)])
def test_full_3x3_layer_channels_last(layout, out_dtype, relu):
    """The 3x3 layer stored channels-last, on the column-group kernel."""
    wl = synth.WORKLOADS["conv3x3_bf16"]
    t = synth.make_inputs(wl)
    y_ref, S = _reference(wl, t, layout)
    got = _run(wl, t, layout, out_dtype, relu, "auto", True)
    _check(got, y_ref, S, relu, out_dtype, TAU["bf16"], False, "full 3x3 %s %s" % (layout, out_dtype))
