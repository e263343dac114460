"""GPU parity: every route of the HIP library against the oracle.

All calls go through the C ABI (ctypes binding).  Sizes: small shapes that span
several tiles with ragged tails, the five full-size workloads (full-tensor
comparison: the oracle finishes them in seconds), integer-valued inputs at the
full sizes (bit-exact), and the degenerate cases (1x1 inputs, pad >= K,
stride > K, a single output channel).
"""
import numpy as np
import pytest
import torch

import oracle
from cnn_convolution_forward_amd import binding as B
from cnn_convolution_forward_amd import synth
from parity import TAU, compare, dev, poisoned, reference, run

pytestmark = pytest.mark.gpu

FULL = ["tiny_f32", "stem_bf16", "conv3x3_bf16", "conv1x1_bf16", "conv3d_bf16",
        "conv3x3_bf16_n8"]          # the 3x3 layer at one GPU's share of an 8-way batch shard


def _routes(wl):
    if wl.dtype == "f32":
        return ["valu"]
    return ["auto", "mfma", "valu", "explicit"]


def _go(wl, t, route):
    return run(wl, t, algo=route if route != "explicit" else "auto", explicit=route == "explicit")


# ---- small shapes: several tiles, ragged edges --------------------------------

SMALL_2D = [
    # (N, C, H, W, Co, K, s, p)
    (3, 20, 13, 17, 70, 3, 1, 1),
    (2, 16, 12, 12, 130, 3, 2, 1),
    (1, 7, 9, 11, 5, 5, 2, 2),
    (2, 33, 7, 6, 64, 1, 1, 0),
    (1, 3, 10, 10, 4, 2, 3, 0),      # stride > K
    (1, 2, 1, 1, 3, 3, 2, 1),        # single-point receptive field
    (1, 4, 3, 3, 9, 1, 1, 2),        # pad > K: fully padded border = bias exactly
    (2, 128, 8, 8, 128, 3, 1, 1),
    (1, 40, 5, 9, 1, 3, 1, 1),       # one output channel
]


@pytest.mark.parametrize("shape", SMALL_2D, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("route", ["mfma", "valu", "explicit"])
@pytest.mark.parametrize("with_bias", [True, False])
def test_small_2d_bf16(shape, route, with_bias):
    N, C, H, W, Co, K, s, p = shape
    wl = synth.Workload("small", 2, N, C, (H, W), Co, K, s, p, "bf16", "normal", 100)
    t = synth.make_inputs(wl, seed=sum(shape), with_bias=with_bias)
    y_ref, S = reference(wl, t)
    compare(_go(wl, t, route), y_ref, S, TAU["bf16"], label="%s %s" % (shape, route))


SMALL_3D = [
    (2, 3, 5, 6, 7, 10, 3, 1, 1),
    (1, 5, 4, 9, 8, 70, 3, 2, 1),
    (1, 16, 3, 4, 5, 33, 1, 1, 0),
    (1, 2, 2, 3, 3, 4, 2, 1, 2),
]


@pytest.mark.parametrize("shape", SMALL_3D, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("route", ["mfma", "valu", "explicit"])
def test_small_3d_bf16(shape, route):
    N, C, D, H, W, Co, K, s, p = shape
    wl = synth.Workload("small3d", 3, N, C, (D, H, W), Co, K, s, p, "bf16", "uniform", 200)
    t = synth.make_inputs(wl, seed=sum(shape))
    y_ref, S = reference(wl, t)
    compare(_go(wl, t, route), y_ref, S, TAU["bf16"], label="%s %s" % (shape, route))


@pytest.mark.parametrize("shape", [(2, 3, 9, 11, 4, 3, 2, 1), (1, 5, 7, 7, 6, 5, 1, 2), (2, 2, 5, 4, 3, 1, 1, 0)])
def test_small_f32(shape):
    N, C, H, W, Co, K, s, p = shape
    wl = synth.Workload("smallf32", 2, N, C, (H, W), Co, K, s, p, "f32", "uniform", 300)
    t = synth.make_inputs(wl, seed=sum(shape))
    y_ref, S = reference(wl, t)
    compare(_go(wl, t, "valu"), y_ref, S, TAU["f32"], label=str(shape))
    wl3 = synth.Workload("smallf32_3d", 3, N, C, (3, H, W), Co, K, s, p, "f32", "uniform", 301)
    t3 = synth.make_inputs(wl3, seed=sum(shape) + 1)
    y_ref, S = reference(wl3, t3)
    compare(_go(wl3, t3, "valu"), y_ref, S, TAU["f32"], label="3d " + str(shape))


# ---- the five workloads (and the sharded 3x3 layer) at full size ---------------

@pytest.mark.parametrize("name", FULL)
def test_full_workload(name):
    wl = synth.ALL_WORKLOADS[name]
    t = synth.make_inputs(wl)
    y_ref, S = reference(wl, t)
    for route in _routes(wl):
        r = compare(_go(wl, t, route), y_ref, S, TAU[wl.dtype], label="%s %s" % (name, route))
        print("%s %s max|d|/S = %.3g" % (name, route, r))


def test_tiny_without_bias():
    wl = synth.WORKLOADS["tiny_f32"]
    t = synth.make_inputs(wl, with_bias=False)
    y_ref, S = reference(wl, t)
    compare(_go(wl, t, "valu"), y_ref, S, TAU["f32"], label="tiny no bias")


@pytest.mark.parametrize("name", FULL)
def test_full_workload_integer_exact(name):
    """x, w in {-2..2}, b in {-3..3}: every partial sum is an exact integer, so
    every route must reproduce the oracle bit for bit (catches any missing or
    misplaced tap)."""
    wl = synth.ALL_WORKLOADS[name]
    t = synth.make_inputs(wl, integer=True)
    y_ref, S = reference(wl, t)
    for route in _routes(wl):
        compare(_go(wl, t, route), y_ref, S, 0, exact=True, label="%s %s int" % (name, route))


# ---- worked examples from the pages -------------------------------------------

def test_pages_worked_examples_on_gpu():
    x = synth.f32_to_bf16_bits(np.arange(25, dtype=np.float32).reshape(1, 1, 5, 5))
    w = synth.f32_to_bf16_bits(np.ones((1, 1, 3, 3), np.float32))
    expect = np.array([[12, 21, 27, 33, 24], [33, 54, 63, 72, 51], [63, 99, 108, 117, 81],
                       [93, 144, 153, 162, 111], [72, 111, 117, 123, 84]], np.float32)
    for algo in ("mfma", "valu"):
        y = B.conv(dev(x, None), dev(w, None), None, 1, 1, algo=algo)
        np.testing.assert_array_equal(y.cpu().numpy()[0, 0], expect)
    x = synth.f32_to_bf16_bits(np.arange(75, dtype=np.float32).reshape(1, 3, 5, 5))
    w = synth.f32_to_bf16_bits(np.ones((2, 3, 3, 3), np.float32))
    for algo in ("mfma", "valu"):
        y = B.conv(dev(x, None), dev(w, None), None, 2, 1, algo=algo).cpu().numpy()
        assert y.shape == (1, 2, 3, 3)
        for oc in range(2):
            np.testing.assert_array_equal(y[0, oc], [[336, 531, 372], [639, 999, 693], [516, 801, 552]])


# ---- explicit X_col: bit-exact copy ------------------------------------------

@pytest.mark.parametrize("shape", [(2, 3, 9, 11, 3, 2, 1), (3, 20, 13, 17, 3, 1, 1), (1, 5, 8, 6, 5, 2, 2),
                                   (2, 7, 5, 5, 1, 1, 0), (1, 2, 4, 4, 2, 3, 3)])
def test_im2col_bit_exact_2d(shape):
    N, C, H, W, K, s, p = shape
    rng = np.random.default_rng(sum(shape))
    x = synth.f32_to_bf16_bits(rng.standard_normal((N, C, H, W)).astype(np.float32))
    col = B.im2col(dev(x, None), K, s, p).cpu().numpy().view(np.uint16)
    ref = oracle.im2col2d(x, K, s, p)
    np.testing.assert_array_equal(oracle.decode(col), ref)


# The vectorised stride-1 path (W % 8 == 0, W_out % 8 == 0): every shift of
# the 16-byte chunks (kw - p from -9 to +2), pads wider than a chunk, and
# K = 1 with no shift at all.
@pytest.mark.parametrize("shape", [(2, 5, 9, 16, 3, 1, 1), (1, 3, 7, 24, 5, 1, 2), (2, 2, 6, 32, 7, 1, 3),
                                   (1, 2, 5, 16, 3, 1, 9), (3, 4, 4, 8, 1, 1, 0), (1, 3, 3, 8, 3, 1, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_im2col_stride1_vector_path_bit_exact(shape):
    N, C, H, W, K, s, p = shape
    assert (W + 2 * p - K + 1) % 8 == 0 and W % 8 == 0
    rng = np.random.default_rng(sum(shape) + 7)
    x = synth.f32_to_bf16_bits(rng.standard_normal((N, C, H, W)).astype(np.float32))
    col = B.im2col(dev(x, None), K, s, p).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.decode(col), oracle.im2col2d(x, K, s, p))


# The explicit route's GEMM on the tiled pointwise kernel (C_in * K^2 % 32 == 0,
# output plane % 8 == 0): ragged output channels and pixel tiles.
@pytest.mark.parametrize("shape", [(2, 32, 12, 16, 70, 3, 1, 1), (3, 64, 8, 24, 128, 3, 1, 1),
                                   (1, 96, 5, 8, 200, 1, 1, 0), (2, 32, 7, 8, 16, 3, 1, 1)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer"])
def test_explicit_pointwise_gemm(shape, integer):
    N, C, H, W, Co, K, s, p = shape
    wl = synth.Workload("xg", 2, N, C, (H, W), Co, K, s, p, "bf16", "normal", 300)
    t = synth.make_inputs(wl, seed=sum(shape), integer=integer)
    y_ref, S = reference(wl, t)
    compare(_go(wl, t, "explicit"), y_ref, S, TAU["bf16"], exact=integer, label="explicit pw %s" % (shape,))


def test_im2col_bit_exact_3d():
    rng = np.random.default_rng(5)
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, 3, 4, 6, 5)).astype(np.float32))
    col = B.im2col(dev(x, None), 3, 1, 1).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.decode(col), oracle.im2col3d(x, 3, 1, 1))


@pytest.mark.parametrize("name", ["stem_bf16", "conv3x3_bf16", "conv1x1_bf16", "conv3d_bf16"])
def test_im2col_full_size_blocks(name):
    """Full-size X_col; the column block of image n depends only on x[n], so the
    oracle checks the first and last image's blocks exactly."""
    wl = synth.WORKLOADS[name]
    t = synth.make_inputs(wl)
    col = B.im2col(dev(t.x, None), wl.K, wl.stride, wl.pad)
    rows = wl.fan_in
    per = int(np.prod(wl.out_spatial()))
    assert tuple(col.shape) == (rows, wl.N * per)
    f = oracle.im2col2d if wl.ndim == 2 else oracle.im2col3d
    for n in (0, wl.N - 1):
        blk = col[:, n * per:(n + 1) * per].cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(oracle.decode(blk), f(t.x[n:n + 1], wl.K, wl.stride, wl.pad))
    del col
    torch.cuda.empty_cache()


# ---- run-to-run determinism and streams ----------------------------------------

@pytest.mark.parametrize("name", ["conv3x3_bf16", "stem_bf16", "conv3d_bf16", "conv1x1_bf16"])
def test_deterministic(name):
    wl = synth.WORKLOADS[name]
    t = synth.make_inputs(wl)
    for route in ("auto", "explicit"):
        a = _go(wl, t, route)
        b = _go(wl, t, route)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), route


def test_runs_on_caller_stream():
    wl = synth.workload("conv3x3_bf16", N=4)
    t = synth.make_inputs(wl)
    y_ref, S = reference(wl, t)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x, w, b = dev(t.x, None), dev(t.w, None), dev(t.b, np.float32)
        y = B.conv(x, w, b, 1, 1)
    s.synchronize()
    compare(y.cpu().numpy(), y_ref, S, TAU["bf16"], label="side stream")


def test_validation_error_leaves_output_untouched():
    x = torch.zeros((1, 3, 5, 5), dtype=torch.int16, device="cuda")
    w = torch.zeros((2, 3, 3, 3), dtype=torch.int16, device="cuda")
    y = poisoned((1, 2, 3, 3))
    st = B.conv2d_fwd_bf16(x.data_ptr(), w.data_ptr(), None, y.data_ptr(), 1, 3, 5, 5, 2, 3, 0, 1, 0, None)
    assert st == 2
    torch.cuda.synchronize()
    assert torch.isnan(y).all()


# ---- the dedicated 3x3 stride-1 kernel across widths, heights and tile plans ----

FAST3x3 = [
    # (N, C, H, W, Co): K=3, s=1, p=1, C % 16 == 0, C >= 32, Co % 128 == 0, W % 8 == 0, W <= 64
    (2, 32, 56, 56, 128),
    (3, 32, 7, 64, 128),
    (1, 32, 8, 8, 256),
    (2, 48, 12, 16, 128),
    (2, 32, 30, 40, 128),
    (1, 32, 5, 24, 128),
    (5, 64, 9, 48, 128),
    (16, 32, 56, 56, 128),     # enough tiles for the chunk-pair plan and the XCD remap
    (2, 16, 56, 56, 128),      # C = 16: one stage (general kernel without a workspace)
    (3, 32, 17, 32, 256),      # W = 32, two channel blocks, ragged last row block
    (1, 16, 8, 56, 128),       # one row block, one stage
]


@pytest.mark.parametrize("shape", FAST3x3, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("ws", [False, True])
def test_conv3x3_fast_kernel(shape, integer, ws):
    """The 3x3 kernel, with weights transposed in the kernel (no workspace) or
    repacked into a workspace first (conv2d_fwd_bf16_ws)."""
    N, C, H, W, Co = shape
    wl = synth.Workload("fast3x3", 2, N, C, (H, W), Co, 3, 1, 1, "bf16", "normal", 400)
    t = synth.make_inputs(wl, seed=sum(shape), integer=integer, with_bias=(sum(shape) % 2 == 0))
    y_ref, S = reference(wl, t)
    x, w, b = dev(t.x, None), dev(t.w, None), dev(t.b, np.float32)
    work = B.workspace_for(x, w, 1, 1, "mfma") if ws else None
    if ws and (C >= 32 or 32 <= W <= 56):
        assert work is not None and work.numel() == Co * C * 9 * 2
    y = poisoned(wl.y_shape)
    B.conv(x, w, b, 1, 1, algo="mfma", out=y, workspace=work)
    torch.cuda.synchronize()
    compare(y.cpu().numpy(), y_ref, S, TAU["bf16"], exact=integer,
            label="%s int=%s ws=%s" % (shape, integer, ws))


@pytest.mark.parametrize("integer", [False, True])
def test_headline_workload_with_workspace(integer):
    wl = synth.WORKLOADS["conv3x3_bf16"]
    t = synth.make_inputs(wl, integer=integer)
    y_ref, S = reference(wl, t)
    x, w, b = dev(t.x, None), dev(t.w, None), dev(t.b, np.float32)
    work = B.workspace_for(x, w, 1, 1)
    for _ in range(2):          # the workspace is rewritten on every call
        y = poisoned(wl.y_shape)
        B.conv(x, w, b, 1, 1, out=y, workspace=work)
        torch.cuda.synchronize()
        compare(y.cpu().numpy(), y_ref, S, TAU["bf16"], exact=integer, label="headline ws int=%s" % integer)


# ---- the pointwise (1x1) kernel: ragged pixel and channel tiles ----------------

POINTWISE = [
    # (ndim, N, C, spatial, Co): K=1, s=1, p=0, C % 32 == 0, plane % 8 == 0
    (2, 3, 64, (9, 8), 200),       # 216 pixels: tiles straddle images, last tile ragged; 2 ragged channel blocks
    (2, 2, 32, (4, 4), 128),       # one partial pixel tile
    (2, 1, 96, (16, 16), 64),      # C_out below one channel block
    (2, 4, 256, (28, 28), 1024),   # the 1x1 workload's layer at N = 4
    (3, 2, 32, (2, 3, 4), 96),     # 3D pointwise
    # the streaming kernel (C in {64, 128, 256}, C_out / 128 dividing 32): the
    # pixels split evenly over 256 / (C_out / 128) contiguous ranges
    (2, 1, 64, (8, 8), 128),       # 64 pixels over 256 ranges: most workgroups have none
    (2, 3, 128, (10, 12), 256),    # 360 pixels over 128 ranges of 0 or 8
    (2, 5, 64, (24, 40), 512),     # ranges of 72 or 80 pixels across image boundaries
]


@pytest.mark.parametrize("shape", POINTWISE, ids=lambda s: "x".join(map(str, s[:3] + s[3] + s[4:])))
@pytest.mark.parametrize("integer", [True, False])
def test_pointwise_kernel(shape, integer):
    ndim, N, C, sp, Co = shape
    wl = synth.Workload("pointwise", ndim, N, C, sp, Co, 1, 1, 0, "bf16", "normal", 500)
    t = synth.make_inputs(wl, seed=N * 1000 + C + Co, integer=integer, with_bias=(Co % 3 != 0))
    y_ref, S = reference(wl, t)
    compare(_go(wl, t, "mfma"), y_ref, S, TAU["bf16"], exact=integer, label="%s int=%s" % (shape, integer))


# ---- the short-reduction kernel (C_in * K^dims <= 128): stems, first 3D layers ---

SMALL_K = [
    # (ndim, N, C, spatial, Co, K, s, p)
    (2, 2, 3, (23, 37), 100, 3, 2, 1),     # stem-like, ragged rows/columns, 2 ragged channel blocks
    (2, 1, 2, (30, 30), 64, 7, 2, 3),      # K = 7 (98 reduction rows)
    (2, 1, 4, (40, 300), 16, 3, 1, 1),     # a wide row: one output row per tile
    (2, 3, 3, (224, 224), 64, 3, 2, 1),    # the stem workload's layer at N = 3
    (2, 2, 33, (7, 6), 64, 1, 1, 0),       # pointwise with C % 32 != 0
    (3, 1, 3, (6, 10, 12), 20, 3, 1, 1),
    (3, 2, 4, (5, 7, 9), 64, 3, 2, 1),     # 108 reduction rows, strided 3D
    (3, 1, 3, (16, 64, 64), 64, 3, 1, 1),  # the 3D workload's layer at N = 1
    (2, 1, 2, (30, 32), 64, 7, 2, 3),      # W % 8 == 0: rows staged in 16-byte pieces, pad 3, K = 7
    (2, 2, 3, (17, 40), 96, 5, 1, 2),      # 16-byte staging, pad 2, ragged rows and channel block
    (3, 2, 4, (5, 8, 16), 64, 3, 2, 1),    # 3D, 16-byte staging, stride 2
    (2, 1, 3, (6, 1024), 64, 3, 1, 1),     # 128 pieces a row: more patch pieces than one batch of loads
    (2, 1, 2, (16, 24), 48, 8, 1, 0),      # 128 reduction rows (the limit), weights 3 pieces a thread
    (3, 1, 1, (4, 6, 16), 32, 5, 1, 2),    # 3D K = 5: 125 rows, K_d = 5 patch planes
    (2, 1, 3, (12, 16), 37, 3, 1, 1),      # 999 weights: a tail past the last 16-byte piece
]


@pytest.mark.parametrize("shape", SMALL_K, ids=lambda s: "x".join(map(str, s[:3] + s[3] + s[4:])))
@pytest.mark.parametrize("integer", [True, False])
def test_small_reduction_kernel(shape, integer):
    ndim, N, C, sp, Co, K, s, p = shape
    wl = synth.Workload("smallk", ndim, N, C, sp, Co, K, s, p, "bf16", "normal", 600)
    t = synth.make_inputs(wl, seed=N * 100 + C * 10 + K, integer=integer, with_bias=(Co % 2 == 0))
    y_ref, S = reference(wl, t)
    compare(_go(wl, t, "auto"), y_ref, S, TAU["bf16"], exact=integer, label="%s int=%s" % (shape, integer))


def test_small_reduction_kernel_misaligned():
    """x and w 2 bytes past a 16-byte boundary: the patch rows go element by
    element and the weights through the element-wise path."""
    wl = synth.Workload("smallk", 2, 2, 3, (20, 24), 64, 3, 1, 1, "bf16", "normal", 601)
    t = synth.make_inputs(wl, seed=601, integer=True)

    def mis(a):
        buf = torch.empty(a.size + 8, dtype=torch.int16, device="cuda")
        v = buf[1:1 + a.size].view(a.shape)
        v.copy_(torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda())
        assert v.data_ptr() % 16 == 2
        return v

    x, w, b = mis(t.x), mis(t.w), dev(t.b, np.float32)
    y = poisoned(wl.y_shape)
    B.conv(x, w, b, 1, 1, out=y)
    torch.cuda.synchronize()
    y_ref, S = reference(wl, t)
    compare(y.cpu().numpy(), y_ref, S, TAU["bf16"], exact=True, label="smallk misaligned")


# ---- packed weights reused across calls (conv2d_pack_weights_bf16 + _prepacked) ----

@pytest.mark.parametrize("shape", [(2, 32, 56, 56, 128), (3, 32, 7, 64, 128), (2, 48, 12, 16, 128),
                                   (1, 16, 9, 40, 256)], ids=lambda s: "x".join(map(str, s)))
def test_pack_once_run_twice(shape):
    """Weights packed once serve two different batches; each result equals the
    oracle and, bit for bit, the one-call workspace path."""
    N, C, H, W, Co = shape
    wl = synth.Workload("prepacked", 2, N, C, (H, W), Co, 3, 1, 1, "bf16", "normal", 700)
    t1 = synth.make_inputs(wl, seed=sum(shape))
    t2 = synth.make_inputs(wl, seed=sum(shape) + 1)
    w, b = dev(t1.w, None), dev(t1.b, np.float32)
    ws = B.pack_weights(w, (N, C, H, W), 1, 1)
    for t in (t1, t2):
        x = dev(t.x, None)
        y = poisoned(wl.y_shape)
        B.conv_prepacked(x, ws, tuple(w.shape), b, 1, 1, out=y)
        y_ws = poisoned(wl.y_shape)
        B.conv(x, w, b, 1, 1, out=y_ws, workspace=B.workspace_for(x, w, 1, 1))
        torch.cuda.synchronize()
        tt = synth.Tensors(x=t.x, w=t1.w, b=t1.b, seed=t.seed)
        y_ref, S = reference(wl, tt)
        compare(y.cpu().numpy(), y_ref, S, TAU["bf16"], label="prepacked %s" % (shape,))
        assert torch.equal(y, y_ws)


# ---- the explicit route's X_col GEMM (direct-to-LDS stage ring): reductions of
# 1 to 18 stages (fewer stages than the ring holds, too), ragged pixel tiles,
# tiles that straddle two images, C_out below, at and above one 128-row block

XCOL_GEMM_2D = [
    # (N, C, H, W, Co, K, s, p): C*K*K % 32 == 0 and N*Ho*Wo % 8 == 0
    (3, 32, 12, 14, 70, 3, 1, 1),     # 9 stages, 504 pixels: last tile 120 wide
    (2, 64, 10, 12, 200, 1, 1, 0),    # 2 stages, two channel blocks, the second ragged
    (1, 32, 8, 8, 256, 1, 1, 0),      # 1 stage
    (4, 32, 16, 16, 128, 3, 2, 1),    # stride 2
    (8, 64, 7, 7, 96, 3, 1, 1),       # plane 49: tiles straddle images; 18 stages
    (4, 32, 16, 16, 256, 1, 1, 0),    # two channel blocks, 8 workgroups: XCD-contiguous block order
    (8, 32, 16, 16, 384, 3, 1, 1),    # three channel blocks, 24 workgroups, XCD-contiguous order
]


@pytest.mark.parametrize("shape", XCOL_GEMM_2D, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("integer", [False, True])
def test_explicit_xcol_gemm(shape, integer):
    N, C, H, W, Co, K, s, p = shape
    wl = synth.Workload("xcolgemm", 2, N, C, (H, W), Co, K, s, p, "bf16", "normal", 400)
    t = synth.make_inputs(wl, seed=sum(shape), integer=integer)
    y_ref, S = reference(wl, t)
    compare(_go(wl, t, "explicit"), y_ref, S, 0 if integer else TAU["bf16"], exact=integer,
            label="%s explicit%s" % (shape, " int" if integer else ""))


def test_explicit_xcol_gemm_3d():
    wl = synth.Workload("xcolgemm3d", 3, 2, 32, (4, 6, 8), 40, 1, 1, 0, "bf16", "uniform", 401)
    t = synth.make_inputs(wl, seed=7)
    y_ref, S = reference(wl, t)
    compare(_go(wl, t, "explicit"), y_ref, S, TAU["bf16"], label="3d explicit")
