"""Pins for the oracle's backward pass (oracle.conv_backward) and col2im.

Each check ties the gradients to something other than the backward loop itself:
  * the forward oracle (pinned in test_oracle_pins*.py) through bilinearity:
    sum(y * dout) = sum(x * dx) = sum(w * dW) for y = conv(x, w) without bias;
  * torch.autograd in float64 on the CPU, including the check of the
    "Hand-writing Conv2D" page (5.3: N=2, C_in=3, 8x10, C_out=4, K=3, s=1,
    p=1, dout = ones);
  * closed forms (all-ones tensors count in-range taps; a single nonzero dout
    scatters the kernel, unflipped, onto its window);
  * the im2col form of the page "Why use matrix multiplication for
    convolution" (3.3): dW_row = dout_col @ X_col^T and dx =
    col2im(W_row^T @ dout_col), with im2col and matmul pinned elsewhere;
  * col2im as the adjoint of im2col, and against torch.nn.functional.fold;
  * the gather (point) form equals the scatter loop element for element.

A plausible mistake (dx overwritten instead of accumulated, dW built from w,
db summed over one image, the stride dropped from the scatter, the group
offset lost, col2im overwriting) fails at least one.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, rng, integer=False):
    if integer:
        return rng.integers(-2, 3, size=shape).astype(np.float64)
    return rng.standard_normal(size=shape)


def _case(ndim, N, C, sp, Co, K, s, p, d, G, rng, integer=False):
    x = _rand((N, C) + tuple(sp), rng, integer)
    w = _rand((Co, C // G) + (K,) * ndim, rng, integer)
    y = oracle.conv_general(x, w, None, s, p, d, G, with_S=False)
    dout = _rand(y.shape, rng, integer)
    return x, w, y, dout


CASES = [
    # (ndim, N, C, spatial, Co, K, s, p, d, G)
    (2, 2, 3, (8, 10), 4, 3, 1, 1, 1, 1),
    (2, 2, 6, (9, 11), 8, 3, 2, 1, 2, 2),
    (2, 1, 4, (12, 7), 4, 3, 1, 2, 2, 4),       # depthwise, dilated
    (2, 3, 5, (7, 9), 6, 5, 3, 4, 1, 1),        # stride 3 > pad windows
    (2, 1, 6, (6, 6), 9, 2, 2, 0, 3, 3),
    (3, 2, 4, (5, 6, 7), 6, 3, 1, 1, 1, 2),
    (3, 1, 3, (6, 5, 7), 3, 3, 2, 2, 2, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:2] + c[2:3] + tuple(c[3]) + c[4:])))
def test_backward_matches_autograd(case):
    ndim, N, C, sp, Co, K, s, p, d, G = case
    rng = np.random.default_rng(sum(sp) + Co + K)
    x, w, _, dout = _case(ndim, N, C, sp, Co, K, s, p, d, G, rng)
    (dx, dw, db), _ = oracle.conv_backward(x, w, dout, s, p, d, G)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.zeros(Co, dtype=torch.float64, requires_grad=True)
    conv = F.conv2d if ndim == 2 else F.conv3d
    conv(xt, wt, bt, stride=s, padding=p, dilation=d, groups=G).backward(torch.tensor(dout))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_pages_backward_check():
    """The page's own check: dout = ones, so the gradients are those of y.sum()
    [Hand-writing Conv2D, 5.3]."""
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((2, 3, 8, 10)), rng.standard_normal((4, 3, 3, 3))
    dout = np.ones((2, 4, 8, 10))
    (dx, dw, db), _ = oracle.conv_backward(x, w, dout, 1, 1)
    xt, wt = torch.tensor(x, requires_grad=True), torch.tensor(w, requires_grad=True)
    bt = torch.zeros(4, dtype=torch.float64, requires_grad=True)
    F.conv2d(xt, wt, bt, stride=1, padding=1).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), atol=1e-12)
    np.testing.assert_array_equal(db, np.full(4, 2 * 8 * 10.0))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:2] + c[2:3] + tuple(c[3]) + c[4:])))
def test_bilinearity_with_forward_oracle(case):
    """sum(y * dout) = sum(x * dx) = sum(w * dW): y is linear in x and in w."""
    ndim, N, C, sp, Co, K, s, p, d, G = case
    rng = np.random.default_rng(7 + sum(sp))
    x, w, y, dout = _case(ndim, N, C, sp, Co, K, s, p, d, G, rng, integer=True)
    (dx, dw, db), _ = oracle.conv_backward(x, w, dout, s, p, d, G)
    e = float(np.sum(y * dout))
    assert float(np.sum(x * dx)) == e
    assert float(np.sum(w * dw)) == e
    # bias: y + b has derivative 1 in b per output position
    np.testing.assert_array_equal(db, dout.sum(axis=tuple(i for i in range(dout.ndim) if i != 1)))


def _valid(o_count, n, K, s, p, d):
    """Per tap k: how many output positions o in [0, o_count) read an in-range input."""
    return np.array([sum(1 for o in range(o_count) if 0 <= o * s + k * d - p < n) for k in range(K)])


@pytest.mark.parametrize("H,W,K,s,p,d", [(7, 9, 3, 1, 1, 1), (8, 6, 3, 2, 2, 2), (5, 5, 5, 1, 4, 1)])
def test_all_ones_closed_forms(H, W, K, s, p, d):
    N, C, Co = 2, 3, 4
    x = np.ones((N, C, H, W))
    w = np.ones((Co, C, K, K))
    Ho, Wo = oracle.out_dim_dilated(H, K, s, p, d), oracle.out_dim_dilated(W, K, s, p, d)
    dout = np.ones((N, Co, Ho, Wo))
    (dx, dw, db), (Sdx, Sdw, Sdb) = oracle.conv_backward(x, w, dout, s, p, d, 1)
    # dW[oc][ic][kh][kw] = N * (#oh whose tap kh lands) * (#ow whose tap kw lands)
    expect_w = N * np.outer(_valid(Ho, H, K, s, p, d), _valid(Wo, W, K, s, p, d))
    for oc, ic in itertools.product(range(Co), range(C)):
        np.testing.assert_array_equal(dw[oc, ic], expect_w)
    # dx[n][ic][ih][iw] = Co * #(oh, kh) hitting ih * #(ow, kw) hitting iw
    hits_h = np.array([sum(1 for oh in range(Ho) for kh in range(K) if oh * s + kh * d - p == i) for i in range(H)])
    hits_w = np.array([sum(1 for ow in range(Wo) for kw in range(K) if ow * s + kw * d - p == i) for i in range(W)])
    for n, ic in itertools.product(range(N), range(C)):
        np.testing.assert_array_equal(dx[n, ic], Co * np.outer(hits_h, hits_w))
    np.testing.assert_array_equal(db, np.full(Co, N * Ho * Wo, np.float64))
    np.testing.assert_array_equal(Sdx, dx)
    np.testing.assert_array_equal(Sdw, dw)
    np.testing.assert_array_equal(Sdb, db)


def test_single_dout_scatters_unflipped_kernel():
    """One nonzero dout at (oh, ow) = (2, 3), s=2, p=1: dx[ih][iw] = w[kh][kw]
    at ih = 2*2 + kh - 1, iw = 3*2 + kw - 1; dW = that window of x."""
    w = np.arange(9, dtype=np.float64).reshape(1, 1, 3, 3) + 1
    x = np.arange(13 * 15, dtype=np.float64).reshape(1, 1, 13, 15)
    dout = np.zeros((1, 1, 7, 8))
    dout[0, 0, 2, 3] = 1.0
    (dx, dw, db), _ = oracle.conv_backward(x, w, dout, 2, 1)
    expect = np.zeros((13, 15))
    expect[3:6, 5:8] = w[0, 0]
    np.testing.assert_array_equal(dx[0, 0], expect)
    np.testing.assert_array_equal(dw[0, 0], x[0, 0, 3:6, 5:8])
    assert db[0] == 1.0


@pytest.mark.parametrize("case", [c for c in CASES if c[9] == 1], ids=lambda c: "x".join(map(str, c[:2] + c[2:3] + tuple(c[3]) + c[4:])))
def test_im2col_form_of_the_gradients(case):
    """dW_row = dout_col @ X_col^T and dx = col2im(W_row^T @ dout_col)
    [Why use matrix multiplication for convolution, 3.3]."""
    ndim, N, C, sp, Co, K, s, p, d, G = case
    rng = np.random.default_rng(3 + Co)
    x, w, _, dout = _case(ndim, N, C, sp, Co, K, s, p, d, G, rng, integer=True)
    (dx, dw, db), _ = oracle.conv_backward(x, w, dout, s, p, d, G)
    col = oracle.im2col_dilated(x, K, s, p, d)                       # (C*K^d, N*plane)
    dout_col = np.moveaxis(dout, 1, 0).reshape(Co, -1)               # (Co, N*plane), columns in output order
    w_row = w.reshape(Co, -1)
    np.testing.assert_array_equal(oracle.matmul(dout_col, col.T.copy()), dw.reshape(Co, -1))
    dcol = oracle.matmul(w_row.T.copy(), dout_col)
    np.testing.assert_array_equal(oracle.col2im_dilated(dcol, x.shape, K, s, p, d), dx)


@pytest.mark.parametrize("shape,K,s,p,d", [((2, 3, 7, 9), 3, 1, 1, 1), ((1, 2, 9, 8), 3, 2, 2, 2),
                                           ((1, 2, 6, 7), 2, 1, 0, 1), ((1, 1, 5, 6), 3, 1, 2, 1)])
def test_col2im_is_adjoint_of_im2col_and_fold(shape, K, s, p, d):
    rng = np.random.default_rng(K + s + p + d)
    x = rng.integers(-3, 4, size=shape).astype(np.float64)
    col = oracle.im2col_dilated(x, K, s, p, d)
    c = rng.integers(-3, 4, size=col.shape).astype(np.float64)
    back = oracle.col2im_dilated(c, shape, K, s, p, d)
    assert float(np.sum(col * c)) == float(np.sum(x * back))
    # torch's fold takes (N, C*K*K, L) per image
    N, L = shape[0], col.shape[1] // shape[0]
    ct = torch.tensor(c.reshape(c.shape[0], N, L).transpose(1, 0, 2).copy())
    ref = F.fold(ct, output_size=shape[2:], kernel_size=K, dilation=d, padding=p, stride=s).numpy()
    np.testing.assert_array_equal(back, ref)


def test_magnitude_sums():
    rng = np.random.default_rng(11)
    x, w, _, dout = _case(2, 2, 4, (7, 8), 6, 3, 2, 1, 1, 2, rng)
    _, (Sdx, Sdw, Sdb) = oracle.conv_backward(x, w, dout, 2, 1, 1, 2)
    (adx, adw, adb), _ = oracle.conv_backward(np.abs(x), np.abs(w), np.abs(dout), 2, 1, 1, 2)
    np.testing.assert_allclose(Sdx, adx, rtol=1e-14)
    np.testing.assert_allclose(Sdw, adw, rtol=1e-14)
    np.testing.assert_allclose(Sdb, adb, rtol=1e-14)


def test_backward_rejects_bad_dout():
    x, w = np.zeros((1, 2, 5, 5)), np.zeros((3, 2, 3, 3))
    with pytest.raises(ValueError):
        oracle.conv_backward(x, w, np.zeros((1, 3, 4, 5)), 1, 1)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:2] + c[2:3] + tuple(c[3]) + c[4:])))
def test_gather_points_equal_scatter(case):
    """The point (gather) form sums the same terms as the scatter loop: with
    integer data every point matches exactly, S included."""
    ndim, N, C, sp, Co, K, s, p, d, G = case
    rng = np.random.default_rng(21 + Co)
    x, w, _, dout = _case(ndim, N, C, sp, Co, K, s, p, d, G, rng, integer=True)
    (dx, dw, db), (Sdx, Sdw, Sdb) = oracle.conv_backward(x, w, dout, s, p, d, G)
    iw = np.arange(dw.size)
    ix = np.arange(dx.size)
    (pdw, pSdw), (pdx, pSdx) = oracle.conv_backward_points(x, w, dout, s, p, d, G, iw, ix)
    np.testing.assert_array_equal(pdw, dw.reshape(-1))
    np.testing.assert_array_equal(pSdw, Sdw.reshape(-1))
    np.testing.assert_array_equal(pdx, dx.reshape(-1))
    np.testing.assert_array_equal(pSdx, Sdx.reshape(-1))
    with pytest.raises(ValueError):
        oracle.conv_backward_points(x, w, dout, s, p, d, G, np.array([dw.size]), np.array([0]))
