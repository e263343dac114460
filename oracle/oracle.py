"""The oracle's Python face: numpy in, numpy out, fp64 throughout.

TEST INFRASTRUCTURE ONLY.  Only tests, the package smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path never does, and this
module imports nothing from the product package.

It wraps ``conv_ref.c`` (built into ``liboracle.so`` by :func:`build`) with ctypes.
Inputs are decoded to float64 here (bf16 bit patterns and fp32 both convert
exactly), so the oracle reads exactly the values the GPU reads.

Citations name the page and its section (see ``conv_ref.c`` for the list).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_ref.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants a mistake in a copy of conv_ref.c points this at the copy's
# build, to show that the pins catch the mistake.
_LIB_OVERRIDE = os.environ.get("CONV_ORACLE_LIB_OVERRIDE")

_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile conv_ref.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(_LIB)
        L.oracle_out_dim.restype = _i64
        L.oracle_out_dim.argtypes = [_i64] * 4
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_void_p, _dp, _i64]
        L.oracle_f32_to_f64.argtypes = [ctypes.c_void_p, _dp, _i64]
        L.oracle_conv2d.restype = ctypes.c_int
        L.oracle_conv2d.argtypes = [_dp, _dp, _dp, _dp, _dp] + [_i64] * 8
        L.oracle_conv3d.restype = ctypes.c_int
        L.oracle_conv3d.argtypes = [_dp, _dp, _dp, _dp, _dp] + [_i64] * 9
        L.oracle_conv_points.restype = ctypes.c_int
        L.oracle_conv_points.argtypes = [ctypes.c_int, _dp, _dp, _dp, ctypes.c_void_p, _i64,
                                         _dp, _dp] + [_i64] * 9
        L.oracle_im2col2d.restype = ctypes.c_int
        L.oracle_im2col2d.argtypes = [_dp, _dp] + [_i64] * 7
        L.oracle_im2col3d.restype = ctypes.c_int
        L.oracle_im2col3d.argtypes = [_dp, _dp] + [_i64] * 8
        L.oracle_matmul.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64]
        L.oracle_out_dim_dilated.restype = _i64
        L.oracle_out_dim_dilated.argtypes = [_i64] * 5
        L.oracle_conv_general.restype = ctypes.c_int
        L.oracle_conv_general.argtypes = [ctypes.c_int, _dp, _dp, _dp, _dp, _dp] + [_i64] * 11
        L.oracle_conv_general_points.restype = ctypes.c_int
        L.oracle_conv_general_points.argtypes = [ctypes.c_int, _dp, _dp, _dp, ctypes.c_void_p, _i64,
                                                 _dp, _dp] + [_i64] * 11
        L.oracle_im2col_dilated.restype = ctypes.c_int
        L.oracle_im2col_dilated.argtypes = [ctypes.c_int, _dp, _dp] + [_i64] * 9
        L.oracle_conv_backward.restype = ctypes.c_int
        L.oracle_conv_backward.argtypes = [ctypes.c_int] + [_dp] * 9 + [_i64] * 11
        L.oracle_conv_backward_points.restype = ctypes.c_int
        L.oracle_conv_backward_points.argtypes = ([ctypes.c_int, _dp, _dp, _dp, ctypes.c_void_p, _i64, _dp, _dp,
                                                   ctypes.c_void_p, _i64, _dp, _dp] + [_i64] * 11)
        L.oracle_round_bf16.restype = ctypes.c_double
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_epilogue.argtypes = [_dp, _dp, _i64, ctypes.c_int, ctypes.c_int]
        L.oracle_conv_nhwc.restype = ctypes.c_int
        L.oracle_conv_nhwc.argtypes = [ctypes.c_int, _dp, _dp, _dp, _dp, _dp] + [_i64] * 11
        L.oracle_winograd_f2x2_3x3.restype = ctypes.c_int
        L.oracle_winograd_f2x2_3x3.argtypes = [_dp, _dp, _dp, _dp, _dp] + [_i64] * 6
        L.oracle_col2im_dilated.restype = ctypes.c_int
        L.oracle_col2im_dilated.argtypes = [ctypes.c_int, _dp, _dp] + [_i64] * 9
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _f64(a):
    """Exact conversion of a float array to a C-contiguous float64 array."""
    return np.ascontiguousarray(a, dtype=np.float64)


def decode(a: np.ndarray) -> np.ndarray:
    """Decode an input tensor to float64 exactly.

    uint16 arrays are taken as bf16 bit patterns; float32/float64 convert directly.
    """
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        out = np.empty(a.shape, np.float64)
        lib().oracle_bf16_to_f64(a.ctypes.data, _p(out), a.size)
        return out
    if a.dtype == np.float32:
        out = np.empty(a.shape, np.float64)
        lib().oracle_f32_to_f64(a.ctypes.data, _p(out), a.size)
        return out
    if a.dtype == np.float64:
        return a
    raise TypeError("oracle inputs are bf16 bits (uint16), float32 or float64, got %s" % a.dtype)


def out_dim(n: int, k: int, s: int, p: int) -> int:
    """floor((n + 2p - k)/s) + 1, or -1 if the window never fits
    [Hand-writing Conv2D, 1.1]."""
    return int(lib().oracle_out_dim(n, k, s, p))


def conv2d(x, w, bias=None, stride=1, pad=0, with_S=True):
    """y (and S = sum |x*w| per output) of a 2D convolution, NCHW x OIHW, fp64
    [Hand-writing Conv2D, 1.1-1.2, 2.1]."""
    x, w = decode(x), decode(w)
    b = None if bias is None else decode(bias)
    N, C, H, W = x.shape
    Co, C2, K, K2 = w.shape
    if C2 != C or K2 != K:
        raise ValueError("weight shape %s does not match C_in=%d with a square kernel" % (w.shape, C))
    if b is not None and b.shape != (Co,):
        raise ValueError("bias must have shape (C_out,)")
    Ho, Wo = out_dim(H, K, stride, pad), out_dim(W, K, stride, pad)
    if Ho < 0 or Wo < 0:
        raise ValueError("kernel larger than padded input")
    y = np.empty((N, Co, Ho, Wo), np.float64)
    S = np.empty_like(y) if with_S else None
    rc = lib().oracle_conv2d(_p(x), _p(w), _p(b), _p(y), _p(S), N, C, H, W, Co, K, stride, pad)
    if rc != 0:
        raise ValueError("oracle_conv2d rejected the shape")
    return (y, S) if with_S else y


def conv3d(x, w, bias=None, stride=1, pad=0, with_S=True):
    """y (and S) of a 3D convolution, NCDHW x (Co, C, K, K, K), fp64
    [PyTorch tensor products and conv2d/conv3d dimension semantics, 5.1-5.2]."""
    x, w = decode(x), decode(w)
    b = None if bias is None else decode(bias)
    N, C, D, H, W = x.shape
    Co, C2, K, K2, K3 = w.shape
    if C2 != C or not (K == K2 == K3):
        raise ValueError("weight shape %s does not match C_in=%d with a cubic kernel" % (w.shape, C))
    Do, Ho, Wo = (out_dim(D, K, stride, pad), out_dim(H, K, stride, pad), out_dim(W, K, stride, pad))
    if min(Do, Ho, Wo) < 0:
        raise ValueError("kernel larger than padded input")
    y = np.empty((N, Co, Do, Ho, Wo), np.float64)
    S = np.empty_like(y) if with_S else None
    rc = lib().oracle_conv3d(_p(x), _p(w), _p(b), _p(y), _p(S), N, C, D, H, W, Co, K, stride, pad)
    if rc != 0:
        raise ValueError("oracle_conv3d rejected the shape")
    return (y, S) if with_S else y


def conv_points(x, w, bias, stride, pad, idx):
    """y and S at the flat output indices ``idx`` only (2D or 3D by x.ndim)."""
    x, w = decode(x), decode(w)
    b = None if bias is None else decode(bias)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    ndim = x.ndim - 2
    if ndim == 2:
        N, C, H, W = x.shape
        D = 1
    else:
        N, C, D, H, W = x.shape
    Co, K = w.shape[0], w.shape[2]
    y = np.empty(idx.shape, np.float64)
    S = np.empty(idx.shape, np.float64)
    rc = lib().oracle_conv_points(ndim, _p(x), _p(w), _p(b), idx.ctypes.data, idx.size,
                                  _p(y), _p(S), N, C, D, H, W, Co, K, stride, pad)
    if rc != 0:
        raise ValueError("oracle_conv_points rejected the request")
    return y, S


def im2col2d(x, K, stride, pad):
    """X_col (C*K*K, N*Ho*Wo) [Why use matrix multiplication for convolution, 2.2, 3.1]."""
    x = decode(x)
    N, C, H, W = x.shape
    Ho, Wo = out_dim(H, K, stride, pad), out_dim(W, K, stride, pad)
    col = np.empty((C * K * K, N * Ho * Wo), np.float64)
    if lib().oracle_im2col2d(_p(x), _p(col), N, C, H, W, K, stride, pad) != 0:
        raise ValueError("bad im2col shape")
    return col


def im2col3d(x, K, stride, pad):
    """X_col (C*K^3, N*Do*Ho*Wo) for NCDHW input."""
    x = decode(x)
    N, C, D, H, W = x.shape
    Do, Ho, Wo = out_dim(D, K, stride, pad), out_dim(H, K, stride, pad), out_dim(W, K, stride, pad)
    col = np.empty((C * K ** 3, N * Do * Ho * Wo), np.float64)
    if lib().oracle_im2col3d(_p(x), _p(col), N, C, D, H, W, K, stride, pad) != 0:
        raise ValueError("bad im2col shape")
    return col


def matmul(A, B):
    """Plain fp64 matrix product [Why use matrix multiplication for convolution, 2.3]."""
    A, B = _f64(A), _f64(B)
    M, Kk = A.shape
    Kk2, Nn = B.shape
    if Kk != Kk2:
        raise ValueError("inner dimensions differ")
    Cm = np.empty((M, Nn), np.float64)
    lib().oracle_matmul(_p(A), _p(B), _p(Cm), M, Kk, Nn)
    return Cm


def out_dim_dilated(n: int, k: int, s: int, p: int, d: int) -> int:
    """floor((n + 2p - d(k-1) - 1)/s) + 1, or -1 if the dilated window never fits
    [PyTorch tensor products and conv2d/conv3d dimension semantics, 4.2]."""
    return int(lib().oracle_out_dim_dilated(n, k, s, p, d))


def _general_dims(x, w, groups):
    ndim = x.ndim - 2
    if ndim == 2:
        N, C, H, W = x.shape
        D = 1
        ks = w.shape[2:]
    elif ndim == 3:
        N, C, D, H, W = x.shape
        ks = w.shape[2:]
    else:
        raise ValueError("x must be NCHW or NCDHW")
    Co, Cg = w.shape[0], w.shape[1]
    if len(ks) != ndim or len(set(ks)) != 1:
        raise ValueError("weight shape %s is not a square/cubic kernel" % (w.shape,))
    if groups < 1 or C % groups or Co % groups or Cg * groups != C:
        raise ValueError("groups=%d does not fit C_in=%d, C_out=%d, weight %s" % (groups, C, Co, w.shape))
    return ndim, N, C, D, H, W, Co, ks[0]


def conv_general(x, w, bias=None, stride=1, pad=0, dilation=1, groups=1, with_S=True):
    """y (and S) of a 2D or 3D convolution with dilation and groups, fp64.
    w: (C_out, C_in/groups, K, K[, K])
    [PyTorch tensor products and conv2d/conv3d dimension semantics, 4.2-4.3, 5.2]."""
    x, w = decode(x), decode(w)
    b = None if bias is None else decode(bias)
    ndim, N, C, D, H, W, Co, K = _general_dims(x, w, groups)
    if b is not None and b.shape != (Co,):
        raise ValueError("bias must have shape (C_out,)")
    sizes = [out_dim_dilated(n, K, stride, pad, dilation) for n in ((D, H, W) if ndim == 3 else (H, W))]
    if min(sizes) < 0:
        raise ValueError("dilated kernel larger than padded input")
    y = np.empty((N, Co) + tuple(sizes), np.float64)
    S = np.empty_like(y) if with_S else None
    rc = lib().oracle_conv_general(ndim, _p(x), _p(w), _p(b), _p(y), _p(S),
                                   N, C, D, H, W, Co, K, stride, pad, dilation, groups)
    if rc != 0:
        raise ValueError("oracle_conv_general rejected the shape")
    return (y, S) if with_S else y


def conv_general_points(x, w, bias, stride, pad, dilation, groups, idx):
    """y and S of conv_general at the flat output indices ``idx`` only."""
    x, w = decode(x), decode(w)
    b = None if bias is None else decode(bias)
    ndim, N, C, D, H, W, Co, K = _general_dims(x, w, groups)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    y = np.empty(idx.shape, np.float64)
    S = np.empty(idx.shape, np.float64)
    rc = lib().oracle_conv_general_points(ndim, _p(x), _p(w), _p(b), idx.ctypes.data, idx.size,
                                          _p(y), _p(S), N, C, D, H, W, Co, K, stride, pad,
                                          dilation, groups)
    if rc != 0:
        raise ValueError("oracle_conv_general_points rejected the request")
    return y, S


def im2col_dilated(x, K, stride, pad, dilation):
    """X_col (C*K^ndim, N*out_plane) with dilated taps, 2D or 3D by x.ndim."""
    x = decode(x)
    ndim = x.ndim - 2
    if ndim == 2:
        N, C, H, W = x.shape
        D = 1
        dims = (H, W)
    else:
        N, C, D, H, W = x.shape
        dims = (D, H, W)
    sizes = [out_dim_dilated(n, K, stride, pad, dilation) for n in dims]
    if min(sizes) < 0:
        raise ValueError("bad im2col shape")
    col = np.empty((C * K ** ndim, N * int(np.prod(sizes))), np.float64)
    if lib().oracle_im2col_dilated(ndim, _p(x), _p(col), N, C, D, H, W, K, stride, pad, dilation) != 0:
        raise ValueError("bad im2col shape")
    return col


def conv_backward(x, w, dout, stride=1, pad=0, dilation=1, groups=1):
    """(dx, dw, db) and their magnitude sums (S_dx, S_dw, S_db) of a 2D or 3D
    convolution, fp64 [Hand-writing Conv2D, 5.1-5.2].  dout has y's shape."""
    x, w, dout = decode(x), decode(w), decode(dout)
    ndim, N, C, D, H, W, Co, K = _general_dims(x, w, groups)
    sizes = [out_dim_dilated(n, K, stride, pad, dilation) for n in ((D, H, W) if ndim == 3 else (H, W))]
    if min(sizes) < 0 or dout.shape != (N, Co) + tuple(sizes):
        raise ValueError("dout shape %s does not match the output (N, C_out) + %s" % (dout.shape, sizes))
    dx, Sdx = np.empty_like(x), np.empty_like(x)
    dw, Sdw = np.empty_like(w), np.empty_like(w)
    db, Sdb = np.empty(Co), np.empty(Co)
    rc = lib().oracle_conv_backward(ndim, _p(x), _p(w), _p(dout), _p(dx), _p(dw), _p(db), _p(Sdx), _p(Sdw),
                                    _p(Sdb), N, C, D, H, W, Co, K, stride, pad, dilation, groups)
    if rc != 0:
        raise ValueError("oracle_conv_backward rejected the shape")
    return (dx, dw, db), (Sdx, Sdw, Sdb)


def conv_backward_points(x, w, dout, stride, pad, dilation, groups, dw_idx, dx_idx):
    """dw and dx (with S) at flat indices only, each summed in gather form
    [Hand-writing Conv2D, 5.1]; for checks at full size."""
    x, w, dout = decode(x), decode(w), decode(dout)
    ndim, N, C, D, H, W, Co, K = _general_dims(x, w, groups)
    dw_idx = np.ascontiguousarray(dw_idx, dtype=np.int64)
    dx_idx = np.ascontiguousarray(dx_idx, dtype=np.int64)
    dw, Sdw = np.empty(dw_idx.shape), np.empty(dw_idx.shape)
    dx, Sdx = np.empty(dx_idx.shape), np.empty(dx_idx.shape)
    rc = lib().oracle_conv_backward_points(ndim, _p(x), _p(w), _p(dout), dw_idx.ctypes.data, dw_idx.size, _p(dw),
                                           _p(Sdw), dx_idx.ctypes.data, dx_idx.size, _p(dx), _p(Sdx),
                                           N, C, D, H, W, Co, K, stride, pad, dilation, groups)
    if rc != 0:
        raise ValueError("oracle_conv_backward_points rejected the request")
    return (dw, Sdw), (dx, Sdx)


def col2im_dilated(col, x_shape, K, stride, pad, dilation=1):
    """Adjoint of im2col_dilated: add each X_col entry onto the input position
    its tap read [Why use matrix multiplication for convolution, 3.3]."""
    col = _f64(col)
    ndim = len(x_shape) - 2
    if ndim == 2:
        N, C, H, W = x_shape
        D = 1
    else:
        N, C, D, H, W = x_shape
    dx = np.empty(tuple(x_shape), np.float64)
    if lib().oracle_col2im_dilated(ndim, _p(col), _p(dx), N, C, D, H, W, K, stride, pad, dilation) != 0:
        raise ValueError("bad col2im shape")
    return dx


def round_bf16(v: float) -> float:
    """Nearest bfloat16 value, ties to even (8-bit significand)."""
    return float(lib().oracle_round_bf16(float(v)))


def epilogue(y, relu=False, to_bf16=False):
    """max(y, 0) if relu, then rounded to bf16 if to_bf16 (fp64 in and out)."""
    y = _f64(y)
    out = np.empty_like(y)
    lib().oracle_epilogue(_p(y), _p(out), y.size, int(bool(relu)), int(bool(to_bf16)))
    return out


def conv_nhwc(x, w, bias=None, stride=1, pad=0, dilation=1, groups=1, with_S=True):
    """The general convolution on channels-last x (N, [D,] H, W, C) -> y
    (N, [Do,] Ho, Wo, Co); w stays (Co, C/groups, K, ...)
    [PyTorch tensor products and conv2d/conv3d dimension semantics, 6.3]."""
    x, w = decode(x), decode(w)
    b = None if bias is None else decode(bias)
    ndim = x.ndim - 2
    if ndim == 2:
        N, H, W, C = x.shape
        D = 1
    elif ndim == 3:
        N, D, H, W, C = x.shape
    else:
        raise ValueError("x must be NHWC or NDHWC")
    Co, Cg, K = w.shape[0], w.shape[1], w.shape[2]
    if w.ndim != ndim + 2 or groups < 1 or Cg * groups != C or Co % groups:
        raise ValueError("weight %s does not fit C_in=%d, groups=%d" % (w.shape, C, groups))
    sizes = [out_dim_dilated(n, K, stride, pad, dilation) for n in ((D, H, W) if ndim == 3 else (H, W))]
    if min(sizes) < 0:
        raise ValueError("dilated kernel larger than padded input")
    y = np.empty((N,) + tuple(sizes) + (Co,), np.float64)
    S = np.empty_like(y) if with_S else None
    rc = lib().oracle_conv_nhwc(ndim, _p(x), _p(w), _p(b), _p(y), _p(S), N, C, D, H, W, Co, K, stride, pad,
                                dilation, groups)
    if rc != 0:
        raise ValueError("oracle_conv_nhwc rejected the shape")
    return (y, S) if with_S else y


def winograd_f2x2_3x3(x, w, bias=None, pad=1):
    """y and Sw of a 3x3, stride-1 convolution by Winograd F(2x2, 3x3) in fp64
    [Why use matrix multiplication for convolution, 5.1]; Sw is the
    transform-domain magnitude sum (see conv_ref.c)."""
    x, w = decode(x), decode(w)
    b = None if bias is None else decode(bias)
    N, C, H, W = x.shape
    Co = w.shape[0]
    if w.shape != (Co, C, 3, 3):
        raise ValueError("Winograd F(2x2,3x3) takes (C_out, C_in, 3, 3) weights")
    Ho, Wo = out_dim(H, 3, 1, pad), out_dim(W, 3, 1, pad)
    if Ho < 0 or Wo < 0:
        raise ValueError("kernel larger than padded input")
    y = np.empty((N, Co, Ho, Wo), np.float64)
    Sw = np.empty_like(y)
    if lib().oracle_winograd_f2x2_3x3(_p(x), _p(w), _p(b), _p(y), _p(Sw), N, C, H, W, Co, pad) != 0:
        raise ValueError("oracle_winograd_f2x2_3x3 rejected the shape")
    return y, Sw


def num_threads() -> int:
    return int(lib().oracle_num_threads())
