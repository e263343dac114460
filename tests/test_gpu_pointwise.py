"""GPU parity of the streaming pointwise kernel (K = 1, NCHW, C_in in {64, 128,
256}, C_out a multiple of 128 with C_out / 128 dividing 32): one persistent
workgroup per CU walks a fixed list of 128-pixel tiles with its block of
weights resident in LDS.

The shapes put every part of that schedule on the test: one and several
tiles per workgroup, tiles straddling two images, a ragged last tile and a
lone partial tile, channel blocks from 1 to 32 (so 256 down to 8 tile
streams), each supported C_in, and a 3D pointwise layer.  Integer-valued
inputs must match the oracle bit for bit; normal inputs within
tau * S.  The bf16 / ReLU epilogues are compared as in the options tests.
"""
import numpy as np
import pytest
import torch

import oracle
from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import TAU, compare, dev, reference, run

pytestmark = pytest.mark.gpu

STREAM = [
    # (ndim, N, C, spatial, Co): pixels P = N * plane, 128-pixel tiles, streams 256 / (Co / 128)
    (2, 5, 64, (80, 84), 128),      # 1 block, 256 streams, 263 tiles (ragged): streams 0..6 take two
    (2, 24, 128, (28, 28), 256),    # 2 blocks, 128 streams, 147 tiles
    (2, 9, 256, (28, 28), 1024),    # 8 blocks, 32 streams, 56 tiles (ragged): streams 0..23 take two
    (2, 5, 256, (9, 8), 4096),      # 32 blocks, 8 streams, 3 tiles straddling images
    (2, 1, 128, (4, 8), 128),       # one partial tile (32 pixels)
    (3, 2, 64, (4, 6, 8), 256),     # 3D pointwise, 3 tiles
]


def _wl(shape, seed=600):
    ndim, N, C, sp, Co = shape
    return synth.Workload("pointwise", ndim, N, C, sp, Co, 1, 1, 0, "bf16", "normal", seed)


@pytest.mark.parametrize("shape", STREAM, ids=lambda s: "x".join(map(str, s[:3] + s[3] + s[4:])))
@pytest.mark.parametrize("integer", [True, False])
def test_stream_pointwise(shape, integer):
    wl = _wl(shape)
    t = synth.make_inputs(wl, seed=shape[1] * 1000 + shape[2] + shape[4], integer=integer,
                          with_bias=(shape[1] % 2 == 1))
    y_ref, S = reference(wl, t)
    compare(run(wl, t, algo="auto"), y_ref, S, TAU["bf16"], exact=integer, label="%s int=%s" % (shape, integer))


@pytest.mark.parametrize("shape", [STREAM[1], STREAM[3], STREAM[5]],
                         ids=lambda s: "x".join(map(str, s[:3] + s[3] + s[4:])))
@pytest.mark.parametrize("out_dtype,relu", [("f32", True), ("bf16", False), ("bf16", True)])
def test_stream_pointwise_epilogues(shape, out_dtype, relu):
    wl = _wl(shape, seed=601)
    t = synth.make_inputs(wl, seed=7 + shape[2])
    y_ref, S = reference(wl, t)
    y = B.conv_ex(dev(t.x, np.float32), dev(t.w, np.float32), dev(t.b, np.float32), 1, 0, 1, 1, "nchw",
                  out_dtype, relu)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    if out_dtype == "bf16":
        got = synth.bf16_bits_to_f32(got.view(np.uint16))
    got = got.astype(np.float64)
    ref = oracle.epilogue(y_ref, relu=relu)
    bound = TAU["bf16"] * S + (2.0 ** -8 * np.abs(ref) if out_dtype == "bf16" else 0.0)
    bad = np.abs(got - ref) > bound
    assert np.all(np.isfinite(got)) and not bad.any(), "%s %s relu=%s: %d outside the bound" % (
        shape, out_dtype, relu, bad.sum())


@pytest.mark.parametrize("shape", [STREAM[2], STREAM[4]], ids=lambda s: "x".join(map(str, s[:3] + s[3] + s[4:])))
def test_stream_pointwise_integer_epilogue_exact(shape):
    """Integer inputs: bf16 output with ReLU equals the oracle's epilogue bit for bit."""
    wl = _wl(shape, seed=602)
    t = synth.make_inputs(wl, seed=11, integer=True)
    y_ref, _ = reference(wl, t)
    y = B.conv_ex(dev(t.x, np.float32), dev(t.w, np.float32), dev(t.b, np.float32), 1, 0, 1, 1, "nchw", "bf16", True)
    torch.cuda.synchronize()
    got = synth.bf16_bits_to_f32(y.cpu().numpy().view(np.uint16)).astype(np.float64)
    want = oracle.epilogue(y_ref, relu=True, to_bf16=True)
    assert np.array_equal(got, want), "%s: %d differ" % (shape, int((got != want).sum()))


def test_stream_pointwise_repeat_calls():
    """Back-to-back launches on one stream (the tile streams carry no state
    between launches): identical outputs, the second into a poisoned buffer."""
    wl = _wl(STREAM[2], seed=603)
    t = synth.make_inputs(wl, seed=5)
    x, w, b = dev(t.x, np.float32), dev(t.w, np.float32), dev(t.b, np.float32)
    y1 = B.conv(x, w, b, 1, 0)
    y2 = torch.full_like(y1, float("nan"))
    for _ in range(3):
        B.conv(x, w, b, 1, 0, out=y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
