"""bf16 outputs at both alignments of y.  The short-reduction kernel (stem,
3D first layer) lets neighbouring lanes swap one value so that each 4-byte
store writes two adjacent pixels; that form needs W_out even and a 4-byte
aligned y, and otherwise the kernel keeps one 2-byte store per output.  The
streaming pointwise and depthwise kernels store 2 bytes per output at any
alignment.

Each case runs even and odd W_out, y at an aligned address and at one 2
bytes past it, with ragged row and channel tails, on integer-valued inputs,
so the result must equal the oracle's epilogue (optional ReLU, then round to
nearest even) bit for bit.  Bytes around a misaligned y must stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import dev

pytestmark = pytest.mark.gpu

CASES = [
    # (name, (ndim, N, C, spatial, Co, K, stride, pad, groups))
    ("pointwise stream", (2, 3, 64, (16, 24), 256, 1, 1, 0, 1)),
    ("pointwise stream ragged tile", (2, 1, 128, (6, 8), 128, 1, 1, 0, 1)),
    ("depthwise even W", (2, 2, 16, (37, 70), 16, 3, 1, 1, 16)),
    ("depthwise odd W", (2, 2, 16, (37, 31), 32, 3, 1, 1, 16)),
    ("depthwise stride 2 odd W", (2, 1, 8, (41, 69), 8, 3, 2, 1, 8)),
    ("stem even W", (2, 2, 3, (33, 36), 64, 3, 2, 1, 1)),
    ("stem odd W", (2, 2, 3, (33, 37), 40, 3, 2, 1, 1)),
    ("3D short reduction", (3, 1, 3, (5, 12, 14), 64, 3, 1, 1, 1)),
    ("3D short reduction odd W", (3, 1, 3, (5, 12, 13), 24, 3, 1, 1, 1)),
]


def _wl(shape):
    ndim, N, C, sp, Co, K, s, p, G = shape
    return synth.Workload("pairs", ndim, N, C, tuple(sp), Co, K, s, p, "bf16", "normal", 700, groups=G)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("misaligned", [False, True], ids=["aligned", "y+2B"])
@pytest.mark.parametrize("relu", [False, True], ids=["plain", "relu"])
def test_bf16_pairs_exact(case, misaligned, relu):
    name, shape = case
    wl = _wl(shape)
    t = synth.make_inputs(wl, seed=sum(shape[3]) + shape[4], integer=True)
    y_ref, _ = oracle.conv_general(t.x, t.w, t.b, wl.stride, wl.pad, 1, wl.groups)
    want = oracle.epilogue(y_ref, relu=relu, to_bf16=True)
    n = int(np.prod(want.shape))
    off = 1 if misaligned else 0
    buf = torch.full((n + 2,), 0x5A5A, dtype=torch.int16, device="cuda")
    y = buf[off:off + n].view(want.shape)
    B.conv_ex(dev(t.x, np.float32), dev(t.w, np.float32), dev(t.b, np.float32), wl.stride, wl.pad, 1, wl.groups,
              "nchw", "bf16", relu, out=y)
    torch.cuda.synchronize()
    raw = buf.cpu().numpy()
    got = synth.bf16_bits_to_f32(raw[off:off + n].view(np.uint16)).reshape(want.shape).astype(np.float64)
    bad = got != want
    assert not bad.any(), "%s misaligned=%s relu=%s: %d differ; first at %s gpu %r want %r" % (
        name, misaligned, relu, bad.sum(), tuple(np.argwhere(bad)[0]), got[bad][0], want[bad][0])
    guard = np.concatenate([raw[:off], raw[off + n:]])
    assert np.all(guard == 0x5A5A), "%s: bytes outside y were written" % name
