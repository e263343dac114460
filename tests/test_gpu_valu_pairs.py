"""GPU parity for the bf16 VALU route's LDS-staged kernel, which takes two
reduction indices per instruction (v_dot2_f32_bf16 on bf16 tap pairs): NCHW,
groups 1, forced with algo "valu", against the fp64 oracle.

The cases cover odd reduction lengths (the pair's second weight is zero past
the end: 27 for the stem, 81 for the 3D layer), even ones, one and several
64-channel blocks (the last one ragged), the 16-channel block form (C_out <=
16), stride, dilation, 3D, the ReLU and bf16-output epilogues, and
integer-valued inputs, for which every route is exact.
"""
import numpy as np
import pytest
import torch

import oracle
from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import TAU, dev

pytestmark = pytest.mark.gpu

CASES = [
    # (ndim, N, C, spatial, C_out, K, stride, pad, dilation)
    (2, 2, 3, (23, 26), 64, 3, 2, 1, 1),       # stem-like: 27 taps (odd)
    (2, 1, 3, (17, 15), 70, 3, 1, 1, 1),       # two channel blocks, the second of 6
    (2, 2, 3, (12, 13), 10, 3, 1, 1, 1),       # 16-channel block form
    (2, 1, 2, (9, 11), 1, 3, 1, 0, 1),         # one output channel, 18 taps (even)
    (2, 2, 4, (13, 10), 33, 2, 3, 0, 1),       # stride > K, 16 taps
    (2, 1, 3, (19, 21), 64, 3, 1, 2, 2),       # dilation 2
    (3, 1, 3, (6, 9, 10), 64, 3, 1, 1, 1),     # 3D: 81 taps (odd)
    (3, 2, 2, (5, 7, 6), 20, 2, 2, 1, 1),      # 3D stride 2, 16 taps
]


def _wl(c, seed):
    ndim, N, C, sp, Co, K, s, p, d = c
    return synth.Workload("valupairs", ndim, N, C, sp, Co, K, s, p, "bf16", "uniform", seed, dilation=d)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, (c[0], c[1], c[2]) + tuple(c[3]) + c[4:])))
@pytest.mark.parametrize("integer", [False, True])
def test_valu_pairs_plain(case, integer):
    wl = _wl(case, 600 + sum(case[3]))
    t = synth.make_inputs(wl, seed=sum(case[3]) + case[4], integer=integer)
    x, w, b = dev(t.x, np.float32), dev(t.w, np.float32), dev(t.b, np.float32)
    y = torch.full(wl.y_shape, float("nan"), dtype=torch.float32, device="cuda")
    B.conv_general(x, w, b, wl.stride, wl.pad, wl.dilation, 1, algo="valu", out=y)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    ref, S = oracle.conv_general(t.x, t.w, t.b, wl.stride, wl.pad, wl.dilation, 1)
    assert np.all(np.isfinite(got)), "unwritten outputs"
    if integer:
        np.testing.assert_array_equal(got, ref)
    else:
        assert np.all(np.abs(got - ref) <= TAU["bf16"] * S)


@pytest.mark.parametrize("case", CASES[:3] + CASES[6:7], ids=lambda c: "x".join(map(str, (c[0], c[2], c[4]))))
@pytest.mark.parametrize("out_dtype,relu", [("f32", True), ("bf16", False), ("bf16", True)])
def test_valu_pairs_epilogue(case, out_dtype, relu):
    wl = _wl(case, 700 + sum(case[3]))
    t = synth.make_inputs(wl, seed=3 * sum(case[3]) + case[4], integer=True)
    x, w, b = dev(t.x, np.float32), dev(t.w, np.float32), dev(t.b, np.float32)
    y = B.conv_ex(x, w, b, wl.stride, wl.pad, wl.dilation, 1, "nchw", out_dtype, relu, "valu", None)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    if out_dtype == "bf16":
        got = synth.bf16_bits_to_f32(got.view(np.uint16))
    got = got.astype(np.float64)
    ref, _ = oracle.conv_general(t.x, t.w, t.b, wl.stride, wl.pad, wl.dilation, 1)
    want = oracle.epilogue(ref, relu=relu, to_bf16=out_dtype == "bf16")
    np.testing.assert_array_equal(got, want)
