"""GPU parity of the persistent 3x3 column-group kernel (two workgroups per
CU walking 32-channel units: whole 64-channel tiles plus leading and trailing
half tiles) against the oracle.

It serves 3x3 / stride 1 / pad 1 NCHW layers with a packed-weight workspace
when C_in % 16 == 0, C_out % 128 == 0, W % 8 == 0 and 32 <= W <= 64; the
library picks it by itself only for small batches, so these tests force it
(CONVFWD_3X3_PERSISTENT=1, read on every call) to cover its multi-item
schedules too.  The
shapes make workgroups own 0, 1, 2, 3 or 4 units, so that full tiles, half
tiles first and last, a ragged last row band (H % 8 != 0), one-stage and
odd-stage reductions (C_in = 16, 48: the next tile's weights are then copied
after the epilogue), more than eight stages (C_in = 256) and the widest rows
(W = 64, whose epilogue image covers every stage buffer) all occur; every case
also runs on integer data, where the result must equal the oracle bit for
bit.
"""
import numpy as np
import pytest
import torch

from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import TAU, compare, dev, poisoned, reference

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _force_persistent(monkeypatch):
    monkeypatch.setenv("CONVFWD_3X3_PERSISTENT", "1")

# (N, C_in, H, W, C_out)
SHAPES = [
    (1, 128, 8, 56, 128),        # 4 units: four CUs with one half tile each
    (1, 128, 9, 32, 128),        # ragged last band (one row)
    (2, 128, 20, 40, 256),       # 48 units, ragged band of 4 rows
    (20, 128, 56, 56, 128),      # 560 units: 2 or 3 a CU
    (12, 256, 30, 48, 256),      # 16 stages a tile
    (32, 128, 56, 56, 128),      # 896 units: 3 or 4 a CU
    (3, 48, 16, 32, 128),        # 3 stages (odd): next weights after the epilogue
    (2, 16, 16, 64, 128),        # 1 stage, W = 64
    (6, 64, 24, 64, 256),        # W = 64, 4 stages
]


def _wl(N, C, H, W, Co, seed):
    return synth.Workload("p3", 2, N, C, (H, W), Co, 3, 1, 1, "bf16", "normal", seed)


def _run(x, w, b, shape, out_dtype="f32", relu=False):
    N, C, H, W, Co = shape
    if out_dtype == "f32" and not relu:
        y = poisoned((N, Co, H, W))
        B.conv(x, w, b, 1, 1, out=y, workspace=B.workspace_for(x, w, 1, 1))
        torch.cuda.synchronize()
        return y.cpu().numpy()
    ws = B.workspace_ex(tuple(x.shape), tuple(w.shape), 1, 1, out_dtype=out_dtype, relu=relu)
    y = B.conv_ex(x, w, b, 1, 1, out_dtype=out_dtype, relu=relu, workspace=ws)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    if out_dtype == "bf16":
        y = synth.bf16_bits_to_f32(y.view(np.uint16))
    return y


@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_persistent3x3(shape, integer):
    wl = _wl(*shape, seed=90 + shape[0])
    t = synth.make_inputs(wl, integer=integer)
    x, w, b = dev(t.x, None), dev(t.w, None), dev(t.b, np.float32)
    print("persistent3x3", shape, "integer" if integer else "random", flush=True)
    y = _run(x, w, b, shape)
    y_ref, S = reference(wl, t)
    compare(y, y_ref, S, TAU["bf16"], exact=integer, label="persistent3x3 %s int=%s" % (shape, integer))


@pytest.mark.parametrize("shape", [(20, 128, 56, 56, 128), (2, 128, 20, 40, 256)], ids=lambda s: "x".join(map(str, s)))
def test_persistent3x3_no_bias(shape):
    wl = _wl(*shape, seed=7)
    t = synth.make_inputs(wl, integer=True)
    x, w = dev(t.x, None), dev(t.w, None)
    y = _run(x, w, None, shape)
    y_ref, S = reference(wl, synth.Tensors(t.x, t.w, None, t.seed))
    compare(y, y_ref, S, TAU["bf16"], exact=True, label="persistent3x3 no bias %s" % (shape,))


@pytest.mark.parametrize("out_dtype,relu", [("f32", True), ("bf16", False), ("bf16", True)])
def test_persistent3x3_epilogues_integer_exact(out_dtype, relu):
    import oracle
    shape = (20, 128, 56, 56, 128)
    wl = _wl(*shape, seed=11)
    t = synth.make_inputs(wl, integer=True)
    x, w, b = dev(t.x, None), dev(t.w, None), dev(t.b, np.float32)
    y = _run(x, w, b, shape, out_dtype, relu)
    y_ref, _ = reference(wl, t)
    np.testing.assert_array_equal(y.astype(np.float64),
                                  oracle.epilogue(y_ref, relu=relu, to_bf16=(out_dtype == "bf16")))


def test_persistent3x3_deterministic_and_rerun():
    """Two calls in a row (the workspace repacked each time) give the same
    bits; the output buffer is fully rewritten."""
    shape = (32, 128, 56, 56, 128)
    wl = _wl(*shape, seed=12)
    t = synth.make_inputs(wl)
    x, w, b = dev(t.x, None), dev(t.w, None), dev(t.b, np.float32)
    a = _run(x, w, b, shape)
    c = _run(x, w, b, shape)
    np.testing.assert_array_equal(a, c)
