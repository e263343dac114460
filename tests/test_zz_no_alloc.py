"""conv2d_fwd_bf16_noalloc: the entry point that allocates nothing.

It runs conv2d_fwd_bf16_ws's kernels with the packed weights in the library's
own static device array instead of a caller workspace, so its output must be
bit-identical to conv2d_fwd_bf16_ws's on the same inputs (and, through it,
within the bf16 parity bar of the oracle).  Two calls in a row, the second on a
smaller input, show that what the first call left in the shared array does
not leak into the second.  Every call goes through the C ABI with raw
pointers."""
import numpy as np
import pytest
import torch

from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import TAU, compare, dev, poisoned, reference

# Fake, distinct device addresses for validation-only calls (never dereferenced).
X, Wp, BIAS, Y = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _wl(N, C, H, W, Co, K=3, pad=1, seed=5):
    return synth.Workload("na", 2, N, C, (H, W), Co, K, 1, pad, "bf16", "normal", seed)


def _pair(wl, integer=False):
    """Run the no-alloc entry point and conv2d_fwd_bf16_ws on the same device
    inputs; return both outputs (numpy) and the inputs."""
    N, C, (H, W), Co, K, s, p = wl.N, wl.C_in, wl.spatial, wl.C_out, wl.K, wl.stride, wl.pad
    t = synth.make_inputs(wl, integer=integer)
    x, w, b = dev(t.x, None), dev(t.w, None), dev(t.b, np.float32)
    y_na, y_ws = poisoned(wl.y_shape), poisoned(wl.y_shape)
    st = torch.cuda.current_stream().cuda_stream
    r = B.conv2d_fwd_bf16_noalloc(x.data_ptr(), w.data_ptr(), b.data_ptr(), y_na.data_ptr(),
                                  N, C, H, W, Co, K, s, p, 0, st)
    assert r == 0, B.status_str(r)
    need = B.conv2d_fwd_workspace_bytes(N, C, H, W, Co, K, s, p, 0)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    r = B.conv2d_fwd_bf16_ws(x.data_ptr(), w.data_ptr(), b.data_ptr(), y_ws.data_ptr(), ws.data_ptr(), need,
                             N, C, H, W, Co, K, s, p, 0, st)
    assert r == 0, B.status_str(r)
    torch.cuda.synchronize()
    return y_na.cpu().numpy(), y_ws.cpu().numpy(), t, need


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_two_calls():
    # First the 3x3 layer at N = 64 with C_out = 256 (576 KiB of packed
    # weights), then a smaller input whose packed weights (288 KiB) cover only
    # part of what the first call wrote to the shared array.
    big = _wl(64, 128, 56, 56, 256, seed=21)
    small = _wl(2, 128, 20, 40, 128, seed=22)
    y_na, y_ws, t, need = _pair(big)
    assert need == 256 * 128 * 9 * 2
    np.testing.assert_array_equal(y_na, y_ws)
    # the big output against the oracle on sampled output channels
    y_ref, S = reference(_wl(4, 128, 56, 56, 256, seed=21), synth.Tensors(t.x[:4], t.w, t.b, t.seed))
    compare(y_na[:4], y_ref, S, TAU["bf16"], label="noalloc big (first 4 images)")

    y_na, y_ws, t, need = _pair(small, integer=True)
    assert 0 < need < 256 * 128 * 9 * 2
    np.testing.assert_array_equal(y_na, y_ws)
    y_ref, S = reference(small, t)
    compare(y_na, y_ref, S, 0, exact=True, label="noalloc small int")


@pytest.mark.gpu
def test_noalloc_route_without_scratch():
    """A layer whose route packs no weights (1x1) uses no scratch at all and
    still gives conv2d_fwd_bf16_ws's bits."""
    wl = _wl(3, 64, 9, 8, 200, K=1, pad=0, seed=23)
    y_na, y_ws, t, need = _pair(wl)
    assert need == 0
    np.testing.assert_array_equal(y_na, y_ws)
    y_ref, S = reference(wl, t)
    compare(y_na, y_ref, S, TAU["bf16"], label="noalloc 1x1")


def test_noalloc_rejects_beyond_static_scratch():
    """C_out * C_in * 9 * 2 bytes of packed weights above 8 MiB: refused on the
    host with CONV_ERR_SCRATCH before any HIP call (fake pointers)."""
    assert B.conv2d_fwd_workspace_bytes(1, 1024, 32, 32, 512, 3, 1, 1, 0) == 512 * 1024 * 9 * 2
    assert B.conv2d_fwd_bf16_noalloc(X, Wp, BIAS, Y, 1, 1024, 32, 32, 512, 3, 1, 1, 0, None) == 9
    assert "scratch" in B.status_str(9)
    # the ordinary argument checks come first
    assert B.conv2d_fwd_bf16_noalloc(None, Wp, BIAS, Y, 1, 1024, 32, 32, 512, 3, 1, 1, 0, None) == 1
    assert B.conv2d_fwd_bf16_noalloc(X, Wp, BIAS, Y, 1, 0, 32, 32, 512, 3, 1, 1, 0, None) == 2
    assert B.conv2d_fwd_bf16_noalloc(X, Wp, BIAS, Y, 1, 128, 32, 32, 128, 3, 1, 1, 7, None) == 7
