"""Thin ctypes binding to libconvfwd.so (argument marshalling only).

The functions named like the C ABI (``conv2d_fwd_bf16`` ...) take raw device
pointers (ints) and sizes, exactly as declared in ``include/conv_fwd.h``, and
return the status code.  The ``conv2d`` / ``conv3d`` / ``im2col`` helpers take
torch tensors that already live on the GPU, allocate the output with torch
(device memory and streams are all torch is used for), pass pointers and the
current HIP stream, and raise :class:`ConvError` on a non-OK status.  Every
arithmetic step runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libconvfwd.so")

CONV_OK = 0
STATUS_NAMES = {0: "CONV_OK", 1: "CONV_ERR_NULL", 2: "CONV_ERR_PARAM", 3: "CONV_ERR_SHAPE",
                4: "CONV_ERR_OVERFLOW", 5: "CONV_ERR_ALIAS", 6: "CONV_ERR_WORKSPACE",
                7: "CONV_ERR_ALGO", 8: "CONV_ERR_HIP", 9: "CONV_ERR_SCRATCH"}
ALGO = {"auto": 0, "mfma": 1, "valu": 2, "winograd": 3}

# Every symbol include/conv_fwd.h declares.
EXPORTS = ("conv_out_dim", "conv_status_str", "conv_version",
           "conv2d_fwd_bf16", "conv2d_fwd_f32", "conv3d_fwd_bf16", "conv3d_fwd_f32",
           "conv2d_fwd_workspace_bytes", "conv2d_fwd_bf16_ws",
           "conv2d_pack_weights_bf16", "conv2d_fwd_bf16_prepacked", "conv2d_fwd_bf16_noalloc",
           "conv_im2col_bytes", "conv2d_im2col_bf16", "conv3d_im2col_bf16",
           "conv2d_fwd_bf16_explicit", "conv3d_fwd_bf16_explicit",
           "conv_out_dim_dilated", "conv_fwd_bf16", "conv_fwd_f32", "conv_xcol_bytes",
           "conv_im2col_bf16", "conv_fwd_explicit_bf16",
           "conv_bwd_data_workspace_bytes", "conv_bwd_data_bf16",
           "conv_bwd_weight_workspace_bytes", "conv_bwd_weight_bf16",
           "conv_fwd_ex_workspace_bytes", "conv_fwd_ex_bf16", "conv_fwd_ex_f32")

LAYOUT = {"nchw": 0, "nhwc": 1}
OUT_DTYPE = {"f32": 0, "bf16": 1}


class ConvParams(ctypes.Structure):
    """conv_params_t: a general problem (dilation and groups)."""
    _fields_ = [(n, ctypes.c_int) for n in ("ndim", "N", "C_in", "D", "H", "W", "C_out", "K", "stride",
                                             "pad", "dilation", "groups")]


class ConvOptions(ctypes.Structure):
    """conv_options_t: layout of x and y, output dtype, ReLU."""
    _fields_ = [("layout", ctypes.c_int), ("out_dtype", ctypes.c_int), ("relu", ctypes.c_int)]


class ConvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, STATUS_NAMES.get(status, status), status_str(status)))


_lib = None
_vp, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t


def lib():
    """Load libconvfwd.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libconvfwd.so is not built (%s); run "
                              "`python -m cnn_convolution_forward_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.conv_out_dim.restype = _i64
        L.conv_out_dim.argtypes = [_i64] * 4
        L.conv_status_str.restype = ctypes.c_char_p
        L.conv_status_str.argtypes = [_i]
        L.conv_version.restype = _i
        L.conv_version.argtypes = []
        d2 = [_vp, _vp, _vp, _vp] + [_i] * 9 + [_vp]
        d3 = [_vp, _vp, _vp, _vp] + [_i] * 10 + [_vp]
        for name, args in (("conv2d_fwd_bf16", d2), ("conv2d_fwd_f32", d2),
                           ("conv3d_fwd_bf16", d3), ("conv3d_fwd_f32", d3)):
            getattr(L, name).restype = _i
            getattr(L, name).argtypes = args
        L.conv2d_fwd_workspace_bytes.restype = _sz
        L.conv2d_fwd_workspace_bytes.argtypes = [_i] * 9
        L.conv2d_fwd_bf16_ws.restype = _i
        L.conv2d_fwd_bf16_ws.argtypes = [_vp] * 5 + [_sz] + [_i] * 9 + [_vp]
        L.conv2d_pack_weights_bf16.restype = _i
        L.conv2d_pack_weights_bf16.argtypes = [_vp, _vp, _sz] + [_i] * 9 + [_vp]
        L.conv2d_fwd_bf16_prepacked.restype = _i
        L.conv2d_fwd_bf16_prepacked.argtypes = [_vp, _vp, _sz, _vp, _vp] + [_i] * 9 + [_vp]
        L.conv2d_fwd_bf16_noalloc.restype = _i
        L.conv2d_fwd_bf16_noalloc.argtypes = d2
        L.conv_im2col_bytes.restype = _sz
        L.conv_im2col_bytes.argtypes = [_i] * 9
        L.conv2d_im2col_bf16.restype = _i
        L.conv2d_im2col_bf16.argtypes = [_vp, _vp] + [_i] * 7 + [_vp]
        L.conv3d_im2col_bf16.restype = _i
        L.conv3d_im2col_bf16.argtypes = [_vp, _vp] + [_i] * 8 + [_vp]
        L.conv2d_fwd_bf16_explicit.restype = _i
        L.conv2d_fwd_bf16_explicit.argtypes = [_vp] * 5 + [_sz] + [_i] * 8 + [_vp]
        L.conv3d_fwd_bf16_explicit.restype = _i
        L.conv3d_fwd_bf16_explicit.argtypes = [_vp] * 5 + [_sz] + [_i] * 9 + [_vp]
        _pp = ctypes.POINTER(ConvParams)
        L.conv_out_dim_dilated.restype = _i64
        L.conv_out_dim_dilated.argtypes = [_i64] * 5
        for name in ("conv_fwd_bf16", "conv_fwd_f32"):
            getattr(L, name).restype = _i
            getattr(L, name).argtypes = [_pp, _vp, _vp, _vp, _vp, _i, _vp]
        L.conv_xcol_bytes.restype = _sz
        L.conv_xcol_bytes.argtypes = [_pp]
        L.conv_im2col_bf16.restype = _i
        L.conv_im2col_bf16.argtypes = [_pp, _vp, _vp, _vp]
        L.conv_fwd_explicit_bf16.restype = _i
        L.conv_fwd_explicit_bf16.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        for name in ("conv_bwd_data_workspace_bytes", "conv_bwd_weight_workspace_bytes"):
            getattr(L, name).restype = _sz
            getattr(L, name).argtypes = [_pp]
        L.conv_bwd_data_bf16.restype = _i
        L.conv_bwd_data_bf16.argtypes = [_pp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.conv_bwd_weight_bf16.restype = _i
        L.conv_bwd_weight_bf16.argtypes = [_pp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        _po = ctypes.POINTER(ConvOptions)
        L.conv_fwd_ex_workspace_bytes.restype = _sz
        L.conv_fwd_ex_workspace_bytes.argtypes = [_pp, _po, _i]
        L.conv_fwd_ex_bf16.restype = _i
        L.conv_fwd_ex_bf16.argtypes = [_pp, _po, _vp, _vp, _vp, _vp, _vp, _sz, _i, _vp]
        L.conv_fwd_ex_f32.restype = _i
        L.conv_fwd_ex_f32.argtypes = [_pp, _po, _vp, _vp, _vp, _vp, _i, _vp]
        _lib = L
    return _lib


# ---- the C ABI, same names, raw pointers -------------------------------------

def conv_out_dim(n, k, stride, pad):
    return int(lib().conv_out_dim(n, k, stride, pad))


def status_str(status):
    return lib().conv_status_str(int(status)).decode()


def conv_status_str(status):
    return status_str(status)


def conv_version():
    return int(lib().conv_version())


def conv2d_fwd_bf16(x, w, bias, y, N, C_in, H, W, C_out, K, stride, pad, algo=0, stream=None):
    return lib().conv2d_fwd_bf16(x, w, bias, y, N, C_in, H, W, C_out, K, stride, pad, algo, stream)


def conv2d_fwd_f32(x, w, bias, y, N, C_in, H, W, C_out, K, stride, pad, algo=0, stream=None):
    return lib().conv2d_fwd_f32(x, w, bias, y, N, C_in, H, W, C_out, K, stride, pad, algo, stream)


def conv3d_fwd_bf16(x, w, bias, y, N, C_in, D, H, W, C_out, K, stride, pad, algo=0, stream=None):
    return lib().conv3d_fwd_bf16(x, w, bias, y, N, C_in, D, H, W, C_out, K, stride, pad, algo, stream)


def conv3d_fwd_f32(x, w, bias, y, N, C_in, D, H, W, C_out, K, stride, pad, algo=0, stream=None):
    return lib().conv3d_fwd_f32(x, w, bias, y, N, C_in, D, H, W, C_out, K, stride, pad, algo, stream)


def conv2d_fwd_workspace_bytes(N, C_in, H, W, C_out, K, stride, pad, algo=0):
    return int(lib().conv2d_fwd_workspace_bytes(N, C_in, H, W, C_out, K, stride, pad, algo))


def conv2d_pack_weights_bf16(w, ws, ws_bytes, N, C_in, H, W, C_out, K, stride, pad, algo=0, stream=None):
    return lib().conv2d_pack_weights_bf16(w, ws, ws_bytes, N, C_in, H, W, C_out, K, stride, pad, algo, stream)


def conv2d_fwd_bf16_prepacked(x, ws, ws_bytes, bias, y, N, C_in, H, W, C_out, K, stride, pad, algo=0,
                              stream=None):
    return lib().conv2d_fwd_bf16_prepacked(x, ws, ws_bytes, bias, y, N, C_in, H, W, C_out, K, stride, pad,
                                           algo, stream)


def conv2d_fwd_bf16_ws(x, w, bias, y, ws, ws_bytes, N, C_in, H, W, C_out, K, stride, pad, algo=0,
                       stream=None):
    return lib().conv2d_fwd_bf16_ws(x, w, bias, y, ws, ws_bytes, N, C_in, H, W, C_out, K, stride, pad,
                                    algo, stream)


def conv2d_fwd_bf16_noalloc(x, w, bias, y, N, C_in, H, W, C_out, K, stride, pad, algo=0, stream=None):
    return lib().conv2d_fwd_bf16_noalloc(x, w, bias, y, N, C_in, H, W, C_out, K, stride, pad, algo, stream)


def conv_im2col_bytes(ndim, N, C_in, D, H, W, K, stride, pad):
    return int(lib().conv_im2col_bytes(ndim, N, C_in, D, H, W, K, stride, pad))


def conv2d_im2col_bf16(x, xcol, N, C_in, H, W, K, stride, pad, stream=None):
    return lib().conv2d_im2col_bf16(x, xcol, N, C_in, H, W, K, stride, pad, stream)


def conv3d_im2col_bf16(x, xcol, N, C_in, D, H, W, K, stride, pad, stream=None):
    return lib().conv3d_im2col_bf16(x, xcol, N, C_in, D, H, W, K, stride, pad, stream)


def conv2d_fwd_bf16_explicit(x, w, bias, y, ws, ws_bytes, N, C_in, H, W, C_out, K, stride, pad,
                             stream=None):
    return lib().conv2d_fwd_bf16_explicit(x, w, bias, y, ws, ws_bytes, N, C_in, H, W, C_out, K,
                                          stride, pad, stream)


def conv3d_fwd_bf16_explicit(x, w, bias, y, ws, ws_bytes, N, C_in, D, H, W, C_out, K, stride, pad,
                             stream=None):
    return lib().conv3d_fwd_bf16_explicit(x, w, bias, y, ws, ws_bytes, N, C_in, D, H, W, C_out, K,
                                          stride, pad, stream)


def _pref(params):
    return None if params is None else ctypes.byref(params)


def conv_out_dim_dilated(n, k, stride, pad, dilation):
    return int(lib().conv_out_dim_dilated(n, k, stride, pad, dilation))


def conv_fwd_bf16(params, x, w, bias, y, algo=0, stream=None):
    return lib().conv_fwd_bf16(_pref(params), x, w, bias, y, algo, stream)


def conv_fwd_f32(params, x, w, bias, y, algo=0, stream=None):
    return lib().conv_fwd_f32(_pref(params), x, w, bias, y, algo, stream)


def conv_xcol_bytes(params):
    return int(lib().conv_xcol_bytes(_pref(params)))


def conv_im2col_bf16(params, x, xcol, stream=None):
    return lib().conv_im2col_bf16(_pref(params), x, xcol, stream)


def conv_fwd_explicit_bf16(params, x, w, bias, y, ws, ws_bytes, stream=None):
    return lib().conv_fwd_explicit_bf16(_pref(params), x, w, bias, y, ws, ws_bytes, stream)


def conv_bwd_data_workspace_bytes(params):
    return int(lib().conv_bwd_data_workspace_bytes(_pref(params)))


def conv_bwd_data_bf16(params, dout, w, dx, ws, ws_bytes, stream=None):
    return lib().conv_bwd_data_bf16(_pref(params), dout, w, dx, ws, ws_bytes, stream)


def conv_bwd_weight_workspace_bytes(params):
    return int(lib().conv_bwd_weight_workspace_bytes(_pref(params)))


def conv_bwd_weight_bf16(params, x, dout, dw, db, ws, ws_bytes, stream=None):
    return lib().conv_bwd_weight_bf16(_pref(params), x, dout, dw, db, ws, ws_bytes, stream)


def _oref(opts):
    return None if opts is None else ctypes.byref(opts)


def conv_fwd_ex_workspace_bytes(params, opts, algo=0):
    return int(lib().conv_fwd_ex_workspace_bytes(_pref(params), _oref(opts), algo))


def conv_fwd_ex_bf16(params, opts, x, w, bias, y, ws, ws_bytes, algo=0, stream=None):
    return lib().conv_fwd_ex_bf16(_pref(params), _oref(opts), x, w, bias, y, ws, ws_bytes, algo, stream)


def conv_fwd_ex_f32(params, opts, x, w, bias, y, algo=0, stream=None):
    return lib().conv_fwd_ex_f32(_pref(params), _oref(opts), x, w, bias, y, algo, stream)


def make_params(x_shape, w_shape, stride=1, pad=0, dilation=1, groups=1):
    """ConvParams from NC(D)HW input and OI(D)HW weight shapes."""
    ndim = len(x_shape) - 2
    if ndim not in (2, 3) or len(w_shape) != ndim + 2:
        raise ValueError("expected 4-D or 5-D x and a weight of the same rank")
    sp = list(x_shape[2:])
    return ConvParams(ndim, x_shape[0], x_shape[1], sp[0] if ndim == 3 else 1, sp[-2], sp[-1], w_shape[0],
                      w_shape[2], stride, pad, dilation, groups)


# ---- torch-tensor helpers (device memory + stream plumbing only) --------------

def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensor(t, name, dtypes):
    torch = _torch()
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (NCHW / OIHW dense)" % name)
    _ = torch


def _dims(x, w, ndim):
    if x.dim() != ndim + 2 or w.dim() != ndim + 2:
        raise ValueError("expected %d-D x and w, got %s and %s" % (ndim + 2, tuple(x.shape), tuple(w.shape)))
    K = w.shape[2]
    if any(k != K for k in w.shape[2:]):
        raise ValueError("only square/cubic kernels are supported")
    if w.shape[1] != x.shape[1]:
        raise ValueError("w.shape[1]=%d != C_in=%d" % (w.shape[1], x.shape[1]))
    return K


def _out_shape(x, w, stride, pad, ndim):
    K = w.shape[2]
    outs = [conv_out_dim(d, K, stride, pad) for d in x.shape[2:]]
    return (x.shape[0], w.shape[0], *outs)


def workspace_for(x, w, stride=1, pad=0, algo="auto"):
    """A device workspace tensor sized for conv(..., workspace=...) (or None)."""
    torch = _torch()
    if x.dim() != 4 or x.dtype == torch.float32:
        return None
    a = ALGO[algo] if isinstance(algo, str) else int(algo)
    n = conv2d_fwd_workspace_bytes(x.shape[0], x.shape[1], x.shape[2], x.shape[3], w.shape[0],
                                   w.shape[2], stride, pad, a)
    return torch.empty(n, dtype=torch.uint8, device=x.device) if n else None


def conv(x, w, bias=None, stride=1, pad=0, algo="auto", out=None, workspace=None):
    """y = conv(x, w) + bias on the GPU.  x/w: bf16 (torch.bfloat16 or int16/uint16
    bit patterns) or float32, dense NC(D)HW / OI(D)HW; bias float32 or None.
    Returns float32 y.  2D or 3D by x.dim().  `workspace` (2D bf16 only, see
    workspace_for) selects conv2d_fwd_bf16_ws."""
    torch = _torch()
    ndim = x.dim() - 2
    if ndim not in (2, 3):
        raise ValueError("x must be 4-D (NCHW) or 5-D (NCDHW)")
    f32 = x.dtype == torch.float32
    half = (torch.bfloat16, torch.int16, torch.uint16)
    _check_tensor(x, "x", (torch.float32,) if f32 else half)
    _check_tensor(w, "w", (torch.float32,) if f32 else half)
    _check_tensor(bias, "bias", (torch.float32,))
    K = _dims(x, w, ndim)
    shape = _out_shape(x, w, stride, pad, ndim)
    if min(shape[2:]) < 1:
        raise ConvError(3, "conv")
    y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=x.device)
    _check_tensor(y, "out", (torch.float32,))
    a = ALGO[algo] if isinstance(algo, str) else int(algo)
    args = [_ptr(x), _ptr(w), _ptr(bias), _ptr(y), x.shape[0], x.shape[1], *x.shape[2:],
            w.shape[0], K, stride, pad, a, _stream()]
    if ndim == 2 and workspace is not None and not f32:
        wsb = workspace.numel() * workspace.element_size()
        st = conv2d_fwd_bf16_ws(args[0], args[1], args[2], args[3], _ptr(workspace), wsb, *args[4:])
    elif ndim == 2:
        st = (conv2d_fwd_f32 if f32 else conv2d_fwd_bf16)(*args)
    else:
        st = (conv3d_fwd_f32 if f32 else conv3d_fwd_bf16)(*args)
    if st != CONV_OK:
        raise ConvError(st, "conv%dd_fwd" % ndim)
    return y


def pack_weights(w, x_shape, stride=1, pad=0, algo="auto", workspace=None):
    """Pack 2D bf16 weights for conv_prepacked (conv2d_pack_weights_bf16);
    returns the workspace tensor.  x_shape: (N, C_in, H, W) of the inputs the
    packed weights will be used with."""
    torch = _torch()
    _check_tensor(w, "w", (torch.bfloat16, torch.int16, torch.uint16))
    N, C, H, W = x_shape
    a = ALGO[algo] if isinstance(algo, str) else int(algo)
    need = conv2d_fwd_workspace_bytes(N, C, H, W, w.shape[0], w.shape[2], stride, pad, a)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=w.device)
    wsb = workspace.numel() * workspace.element_size()
    st = conv2d_pack_weights_bf16(_ptr(w), _ptr(workspace), wsb, N, C, H, W, w.shape[0], w.shape[2], stride,
                                  pad, a, _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv2d_pack_weights_bf16")
    return workspace


def conv_prepacked(x, workspace, w_shape, bias=None, stride=1, pad=0, algo="auto", out=None):
    """conv(x, w) + bias with w taken from pack_weights' workspace (w_shape:
    the (C_out, C_in, K, K) shape of the packed weights)."""
    torch = _torch()
    _check_tensor(x, "x", (torch.bfloat16, torch.int16, torch.uint16))
    _check_tensor(bias, "bias", (torch.float32,))
    C_out, C_in, K = w_shape[0], w_shape[1], w_shape[2]
    if x.dim() != 4 or x.shape[1] != C_in:
        raise ValueError("x must be N x C_in x H x W with C_in = %d" % C_in)
    outs = [conv_out_dim(d, K, stride, pad) for d in x.shape[2:]]
    if min(outs) < 1:
        raise ConvError(3, "conv_prepacked")
    y = out if out is not None else torch.empty((x.shape[0], C_out, *outs), dtype=torch.float32,
                                                device=x.device)
    _check_tensor(y, "out", (torch.float32,))
    a = ALGO[algo] if isinstance(algo, str) else int(algo)
    wsb = workspace.numel() * workspace.element_size()
    st = conv2d_fwd_bf16_prepacked(_ptr(x), _ptr(workspace), wsb, _ptr(bias), _ptr(y), x.shape[0], C_in,
                                   x.shape[2], x.shape[3], C_out, K, stride, pad, a, _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv2d_fwd_bf16_prepacked")
    return y


def im2col(x, K, stride=1, pad=0, out=None):
    """Explicit X_col (C_in*K^dims, N*prod(out)) as int16 bf16 bit patterns."""
    torch = _torch()
    ndim = x.dim() - 2
    _check_tensor(x, "x", (torch.bfloat16, torch.int16, torch.uint16))
    N, C = x.shape[:2]
    sp = list(x.shape[2:])
    D = sp[0] if ndim == 3 else 1
    nbytes = conv_im2col_bytes(ndim, N, C, D, sp[-2], sp[-1], K, stride, pad)
    if nbytes == 0:
        raise ConvError(2, "conv_im2col_bytes")
    outs = [conv_out_dim(d, K, stride, pad) for d in sp]
    cols = N
    for o in outs:
        cols *= o
    rows = C * K ** ndim
    col = out if out is not None else torch.empty((rows, cols), dtype=torch.int16, device=x.device)
    if ndim == 2:
        st = conv2d_im2col_bf16(_ptr(x), _ptr(col), N, C, sp[0], sp[1], K, stride, pad, _stream())
    else:
        st = conv3d_im2col_bf16(_ptr(x), _ptr(col), N, C, D, sp[1], sp[2], K, stride, pad, _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv%dd_im2col_bf16" % ndim)
    return col


def conv_explicit(x, w, bias=None, stride=1, pad=0, workspace=None, out=None):
    """im2col into a workspace, then the MFMA GEMM; returns float32 y."""
    torch = _torch()
    ndim = x.dim() - 2
    half = (torch.bfloat16, torch.int16, torch.uint16)
    _check_tensor(x, "x", half)
    _check_tensor(w, "w", half)
    _check_tensor(bias, "bias", (torch.float32,))
    K = _dims(x, w, ndim)
    N, C = x.shape[:2]
    sp = list(x.shape[2:])
    D = sp[0] if ndim == 3 else 1
    nbytes = conv_im2col_bytes(ndim, N, C, D, sp[-2], sp[-1], K, stride, pad)
    if nbytes == 0:
        raise ConvError(2, "conv_im2col_bytes")
    ws = workspace if workspace is not None else torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    shape = _out_shape(x, w, stride, pad, ndim)
    y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=x.device)
    wsb = ws.numel() * ws.element_size()
    if ndim == 2:
        st = conv2d_fwd_bf16_explicit(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), _ptr(ws), wsb, N, C,
                                      sp[0], sp[1], w.shape[0], K, stride, pad, _stream())
    else:
        st = conv3d_fwd_bf16_explicit(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), _ptr(ws), wsb, N, C,
                                      D, sp[1], sp[2], w.shape[0], K, stride, pad, _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv%dd_fwd_bf16_explicit" % ndim)
    return y


def _general_out_shape(x, w, stride, pad, dilation):
    K = w.shape[2]
    outs = [conv_out_dim_dilated(d, K, stride, pad, dilation) for d in x.shape[2:]]
    return (x.shape[0], w.shape[0], *outs)


def _general_check(x, w, groups, half_ok=True):
    torch = _torch()
    ndim = x.dim() - 2
    if ndim not in (2, 3) or w.dim() != x.dim():
        raise ValueError("x must be 4-D or 5-D and w of the same rank")
    if any(k != w.shape[2] for k in w.shape[2:]):
        raise ValueError("only square/cubic kernels are supported")
    if groups < 1 or x.shape[1] % groups or w.shape[0] % groups or w.shape[1] * groups != x.shape[1]:
        raise ValueError("w.shape[1]=%d * groups=%d must equal C_in=%d and groups must divide C_out=%d"
                         % (w.shape[1], groups, x.shape[1], w.shape[0]))
    _ = torch
    return ndim


def conv_general(x, w, bias=None, stride=1, pad=0, dilation=1, groups=1, algo="auto", out=None):
    """y = conv(x, w) + bias with dilation and groups (conv_fwd_bf16 /
    conv_fwd_f32).  w: (C_out, C_in/groups, K, K[, K]).  Returns float32 y."""
    torch = _torch()
    _general_check(x, w, groups)
    f32 = x.dtype == torch.float32
    half = (torch.bfloat16, torch.int16, torch.uint16)
    _check_tensor(x, "x", (torch.float32,) if f32 else half)
    _check_tensor(w, "w", (torch.float32,) if f32 else half)
    _check_tensor(bias, "bias", (torch.float32,))
    shape = _general_out_shape(x, w, stride, pad, dilation)
    if min(shape[2:]) < 1:
        raise ConvError(3, "conv_general")
    y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=x.device)
    _check_tensor(y, "out", (torch.float32,))
    prm = make_params(tuple(x.shape), tuple(w.shape), stride, pad, dilation, groups)
    a = ALGO[algo] if isinstance(algo, str) else int(algo)
    fn = conv_fwd_f32 if f32 else conv_fwd_bf16
    st = fn(prm, _ptr(x), _ptr(w), _ptr(bias), _ptr(y), a, _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv_fwd_f32" if f32 else "conv_fwd_bf16")
    return y


def im2col_general(x, K, stride=1, pad=0, dilation=1, out=None):
    """X_col with dilated taps (conv_im2col_bf16) as int16 bf16 bit patterns."""
    torch = _torch()
    _check_tensor(x, "x", (torch.bfloat16, torch.int16, torch.uint16))
    ndim = x.dim() - 2
    prm = make_params(tuple(x.shape), (1, x.shape[1]) + (K,) * ndim, stride, pad, dilation, 1)
    nbytes = conv_xcol_bytes(prm)
    if nbytes == 0:
        raise ConvError(2, "conv_xcol_bytes")
    rows = x.shape[1] * K ** ndim
    col = out if out is not None else torch.empty((rows, nbytes // 2 // rows), dtype=torch.int16,
                                                  device=x.device)
    st = conv_im2col_bf16(prm, _ptr(x), _ptr(col), _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv_im2col_bf16")
    return col


def conv_explicit_general(x, w, bias=None, stride=1, pad=0, dilation=1, groups=1, workspace=None, out=None):
    """conv_fwd_explicit_bf16: dilated im2col into a workspace, then one GEMM per group."""
    torch = _torch()
    _general_check(x, w, groups)
    half = (torch.bfloat16, torch.int16, torch.uint16)
    _check_tensor(x, "x", half)
    _check_tensor(w, "w", half)
    _check_tensor(bias, "bias", (torch.float32,))
    prm = make_params(tuple(x.shape), tuple(w.shape), stride, pad, dilation, groups)
    nbytes = conv_xcol_bytes(prm)
    if nbytes == 0:
        raise ConvError(2, "conv_xcol_bytes")
    ws = workspace if workspace is not None else torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    shape = _general_out_shape(x, w, stride, pad, dilation)
    y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=x.device)
    st = conv_fwd_explicit_bf16(prm, _ptr(x), _ptr(w), _ptr(bias), _ptr(y), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv_fwd_explicit_bf16")
    return y


def conv_backward(x, w, dout, stride=1, pad=0, dilation=1, groups=1, with_db=True, out=None):
    """(dx, dw, db) of y = conv(x, w) + b for upstream gradient dout, all bf16
    inputs (conv_bwd_data_bf16 + conv_bwd_weight_bf16); fp32 results.  `out`:
    optional (dx, dw, db) tensors to write into."""
    torch = _torch()
    _general_check(x, w, groups)
    half = (torch.bfloat16, torch.int16, torch.uint16)
    for t, n in ((x, "x"), (w, "w"), (dout, "dout")):
        _check_tensor(t, n, half)
    prm = make_params(tuple(x.shape), tuple(w.shape), stride, pad, dilation, groups)
    yshape = _general_out_shape(x, w, stride, pad, dilation)
    if tuple(dout.shape) != tuple(yshape):
        raise ValueError("dout has shape %s, the output is %s" % (tuple(dout.shape), yshape))
    if out is None:
        dx = torch.empty(x.shape, dtype=torch.float32, device=x.device)
        dw = torch.empty(w.shape, dtype=torch.float32, device=x.device)
        db = torch.empty((w.shape[0],), dtype=torch.float32, device=x.device) if with_db else None
    else:
        dx, dw, db = out
    nd, nw = conv_bwd_data_workspace_bytes(prm), conv_bwd_weight_workspace_bytes(prm)
    wsd = torch.empty(max(nd, 16), dtype=torch.uint8, device=x.device)
    wsw = torch.empty(max(nw, 16), dtype=torch.uint8, device=x.device)
    st = conv_bwd_data_bf16(prm, _ptr(dout), _ptr(w), _ptr(dx), _ptr(wsd), wsd.numel(), _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv_bwd_data_bf16")
    st = conv_bwd_weight_bf16(prm, _ptr(x), _ptr(dout), _ptr(dw), _ptr(db), _ptr(wsw), wsw.numel(), _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv_bwd_weight_bf16")
    return dx, dw, db


def conv_ex(x, w, bias=None, stride=1, pad=0, dilation=1, groups=1, layout="nchw", out_dtype="f32", relu=False,
            algo="auto", workspace=None, out=None):
    """conv_fwd_ex_bf16 / conv_fwd_ex_f32.  layout "nhwc": x is (N, [D,] H, W, C)
    and y comes back (N, [D,] H, W, C_out); w stays (C_out, C_in/groups, K...).
    out_dtype "bf16": y holds bf16 bits (int16).  workspace: a tensor from
    workspace_ex() (packed 3x3 weights) or None."""
    torch = _torch()
    f32 = x.dtype == torch.float32
    half = (torch.bfloat16, torch.int16, torch.uint16)
    _check_tensor(x, "x", (torch.float32,) if f32 else half)
    _check_tensor(w, "w", (torch.float32,) if f32 else half)
    _check_tensor(bias, "bias", (torch.float32,))
    if layout == "nhwc":
        logical = (x.shape[0], x.shape[-1]) + tuple(x.shape[1:-1])
    else:
        logical = tuple(x.shape)
    prm = make_params(logical, tuple(w.shape), stride, pad, dilation, groups)
    opts = ConvOptions(LAYOUT[layout], OUT_DTYPE[out_dtype], int(bool(relu)))
    K = w.shape[2]
    outs = [conv_out_dim_dilated(d, K, stride, pad, dilation) for d in logical[2:]]
    if min(outs) < 1:
        raise ConvError(3, "conv_ex")
    shape = (logical[0], *outs, w.shape[0]) if layout == "nhwc" else (logical[0], w.shape[0], *outs)
    dt = torch.float32 if out_dtype == "f32" else torch.int16
    y = out if out is not None else torch.empty(shape, dtype=dt, device=x.device)
    a = ALGO[algo] if isinstance(algo, str) else int(algo)
    if f32:
        st = conv_fwd_ex_f32(prm, opts, _ptr(x), _ptr(w), _ptr(bias), _ptr(y), a, _stream())
    else:
        wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
        st = conv_fwd_ex_bf16(prm, opts, _ptr(x), _ptr(w), _ptr(bias), _ptr(y), _ptr(workspace), wsb, a, _stream())
    if st != CONV_OK:
        raise ConvError(st, "conv_fwd_ex")
    return y


def workspace_ex(x_shape, w_shape, stride=1, pad=0, dilation=1, groups=1, layout="nchw", out_dtype="f32",
                 relu=False, algo="auto", device="cuda"):
    """Workspace tensor for conv_ex (None when no route uses one); x_shape logical NC(D)HW."""
    torch = _torch()
    prm = make_params(tuple(x_shape), tuple(w_shape), stride, pad, dilation, groups)
    opts = ConvOptions(LAYOUT[layout], OUT_DTYPE[out_dtype], int(bool(relu)))
    a = ALGO[algo] if isinstance(algo, str) else int(algo)
    n = conv_fwd_ex_workspace_bytes(prm, opts, a)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None
