"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, computes output sizes like the pages' formula, and rejects
every invalid argument before any HIP call (so no kernel is ever launched
here: all pointers below are fake and never dereferenced)."""
import ctypes
import json
import os
import re

import pytest

from cnn_convolution_forward_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv_fwd.h")

# Fake, distinct, non-overlapping "device" addresses for validation-only calls.
X, Wp, BIAS, Y, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def declared_symbols():
    text = open(HEADER).read()
    text = text.split("#define CONV_API", 1)[1]
    return sorted(set(re.findall(r"CONV_API\s+[\w\s\*]*?\b(\w+)\s*\(", text)))


def test_header_declares_binding_exports():
    assert declared_symbols() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    out = os.popen("nm -D --defined-only %s" % B.LIB_PATH).read()
    exported = set(re.findall(r" T (\w+)", out))
    assert set(declared_symbols()) == exported


def test_version_and_status_strings():
    assert B.conv_version() >= 100
    for s in range(10):
        assert B.status_str(s) and B.status_str(s) != "unknown status"
    assert B.status_str(99) == "unknown status"


def test_out_dim_matches_page_table(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "output_sizes.json")))
    for c in g["cases"]:
        assert B.conv_out_dim(c["in"], c["k"], c["s"], c["p"]) == c["out"], c
    assert B.conv_out_dim(5, 3, 0, 1) == -1
    assert B.conv_out_dim(5, 3, 1, -1) == -1


def _c2(x=X, w=Wp, b=BIAS, y=Y, N=2, C=3, H=9, W=11, Co=4, K=3, s=2, p=1, algo=0):
    return B.conv2d_fwd_bf16(x, w, b, y, N, C, H, W, Co, K, s, p, algo, None)


def test_null_pointers():
    assert _c2(x=None) == 1
    assert _c2(w=None) == 1
    assert _c2(y=None) == 1
    assert B.conv2d_fwd_f32(X, None, None, Y, 2, 3, 9, 11, 4, 3, 2, 1, 0, None) == 1
    assert B.conv2d_im2col_bf16(None, Y, 2, 3, 9, 11, 3, 2, 1, None) == 1
    assert B.conv2d_fwd_bf16_explicit(X, Wp, None, Y, None, 1 << 20, 2, 3, 9, 11, 4, 3, 2, 1, None) == 1


@pytest.mark.parametrize("kw", [dict(N=0), dict(C=0), dict(H=0), dict(W=-1), dict(Co=0), dict(K=0),
                                dict(s=0), dict(s=-2), dict(p=-1)])
def test_bad_params(kw):
    assert _c2(**kw) == 2


def test_kernel_larger_than_padded_input():
    assert _c2(H=1, W=1, K=3, s=1, p=0) == 3
    assert _c2(H=5, W=1, K=3, s=1, p=0) == 3
    assert B.conv3d_fwd_bf16(X, Wp, BIAS, Y, 1, 1, 1, 5, 5, 1, 3, 1, 0, 0, None) == 3
    # pad >= K is legal (fully padded border windows)
    assert B.conv_im2col_bytes(2, 1, 1, 1, 1, 1, 1, 1, 2) == 25 * 2


def test_overflow_rejected():
    # x with 2^31 elements
    assert _c2(N=2, C=1024, H=1024, W=1024, Co=1, K=1, s=1, p=0) == 4
    # y with >= 2^31 elements while x is small
    assert _c2(N=1, C=1, H=46341, W=46341, Co=1, K=1, s=1, p=0) == 4
    assert B.conv_im2col_bytes(2, 64, 128, 1, 256, 256, 3, 1, 1) == 0     # X_col >= 2^31


def test_alias_rejected():
    assert _c2(y=X) == 5
    assert _c2(y=X + 16) == 5
    assert _c2(y=BIAS - 8) == 5
    assert _c2(y=Wp + 2) == 5
    ws_bytes = B.conv_im2col_bytes(2, 2, 3, 1, 9, 11, 3, 2, 1)
    assert B.conv2d_fwd_bf16_explicit(X, Wp, None, Y, Y + 4, ws_bytes, 2, 3, 9, 11, 4, 3, 2, 1, None) == 5
    assert B.conv2d_fwd_bf16_explicit(X, Wp, None, Y, X, ws_bytes, 2, 3, 9, 11, 4, 3, 2, 1, None) == 5


def test_bad_algo():
    assert _c2(algo=3) == 7
    assert _c2(algo=-1) == 7
    assert B.conv2d_fwd_f32(X, Wp, BIAS, Y, 2, 3, 9, 11, 4, 3, 2, 1, 1, None) == 7   # MFMA is bf16-only


def test_workspace_size():
    need = B.conv_im2col_bytes(2, 2, 3, 1, 9, 11, 3, 2, 1)
    assert need == 27 * (2 * 5 * 6) * 2
    assert B.conv2d_fwd_bf16_explicit(X, Wp, None, Y, WS, need - 1, 2, 3, 9, 11, 4, 3, 2, 1, None) == 6
    assert B.conv_im2col_bytes(3, 8, 3, 16, 64, 64, 3, 1, 1) == 81 * 8 * 16 * 64 * 64 * 2
    assert B.conv_im2col_bytes(4, 8, 3, 16, 64, 64, 3, 1, 1) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        B.lib()


def test_workspace_entry_point_validation():
    need = B.conv2d_fwd_workspace_bytes(64, 128, 56, 56, 128, 3, 1, 1, 0)
    assert need == 128 * 128 * 9 * 2
    assert B.conv2d_fwd_workspace_bytes(64, 128, 56, 56, 128, 3, 1, 1, 2) == 0     # VALU route
    assert B.conv2d_fwd_workspace_bytes(2, 3, 9, 11, 4, 3, 2, 1, 0) == 0          # no route needs one
    assert B.conv2d_fwd_workspace_bytes(2, 16, 56, 56, 128, 3, 1, 1, 0) == 128 * 16 * 9 * 2   # one stage
    assert B.conv2d_fwd_workspace_bytes(2, 16, 9, 12, 128, 3, 1, 1, 0) == 0       # W = 12: general kernel
    args = (64, 128, 56, 56, 128, 3, 1, 1, 0, None)
    assert B.conv2d_fwd_bf16_ws(X, Wp, BIAS, Y, None, 0, *args) == 6
    assert B.conv2d_fwd_bf16_ws(X, Wp, BIAS, Y, WS, need - 2, *args) == 6
    assert B.conv2d_fwd_bf16_ws(X, Wp, BIAS, Y, WS + 8, need, *args) == 6          # misaligned
    assert B.conv2d_fwd_bf16_ws(X, Wp, BIAS, Y, Y + 64, need, *args) == 5          # overlaps y
    assert B.conv2d_fwd_bf16_ws(X, Wp, BIAS, Y, WS, need, 64, 128, 56, 56, 128, 3, 1, 1, 5, None) == 7


def test_pack_and_prepacked_validation():
    """Host-side checks of the pack / prepacked pair (no GPU call is reached)."""
    need = B.conv2d_fwd_workspace_bytes(64, 128, 56, 56, 128, 3, 1, 1, 0)
    dims = (64, 128, 56, 56, 128, 3, 1, 1)
    assert B.conv2d_pack_weights_bf16(None, WS, need, *dims, 0, None) == 1          # NULL w
    assert B.conv2d_pack_weights_bf16(Wp, None, need, *dims, 0, None) == 1          # NULL workspace
    assert B.conv2d_pack_weights_bf16(Wp, WS, need, 64, 128, 56, 56, 128, 0, 1, 1, 0, None) == 2
    assert B.conv2d_pack_weights_bf16(Wp, WS, need, *dims, 2, None) == 7            # VALU: nothing packed
    assert B.conv2d_pack_weights_bf16(Wp, WS, need, 2, 3, 9, 11, 4, 3, 2, 1, 0, None) == 7   # no packed route
    assert B.conv2d_pack_weights_bf16(Wp, WS, need - 2, *dims, 0, None) == 6
    assert B.conv2d_pack_weights_bf16(Wp, WS + 8, need, *dims, 0, None) == 6        # misaligned workspace
    assert B.conv2d_pack_weights_bf16(Wp, Wp, need, *dims, 0, None) == 5            # workspace over w
    assert B.conv2d_pack_weights_bf16(Wp + 2, WS, need, *dims, 0, None) == 7        # misaligned w
    assert B.conv2d_fwd_bf16_prepacked(None, WS, need, BIAS, Y, *dims, 0, None) == 1
    assert B.conv2d_fwd_bf16_prepacked(X, None, need, BIAS, Y, *dims, 0, None) == 1
    assert B.conv2d_fwd_bf16_prepacked(X, WS, need, BIAS, None, *dims, 0, None) == 1
    assert B.conv2d_fwd_bf16_prepacked(X, WS, need, BIAS, Y, *dims, 7, None) == 7
    assert B.conv2d_fwd_bf16_prepacked(X, WS, need, BIAS, Y, 2, 3, 9, 11, 4, 3, 2, 1, 0, None) == 7
    assert B.conv2d_fwd_bf16_prepacked(X, WS, need - 16, BIAS, Y, *dims, 0, None) == 6
    assert B.conv2d_fwd_bf16_prepacked(X, WS, need, BIAS, WS + 64, *dims, 0, None) == 5   # y over workspace
    assert B.conv2d_fwd_bf16_prepacked(X, WS, need, BIAS, X + 64, *dims, 0, None) == 5    # y over x


# ---- general entry points (dilation and groups) ------------------------------

def _gp(**kw):
    base = dict(ndim=2, N=2, C_in=8, D=1, H=9, W=11, C_out=16, K=3, stride=1, pad=1, dilation=2, groups=4)
    base.update(kw)
    return B.ConvParams(**base)


def test_out_dim_dilated_matches_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "dilated_sizes.json")))
    for c in g["cases"]:
        assert B.conv_out_dim_dilated(c["in"], c["k"], c["s"], c["p"], c["d"]) == c["out"], c
    g = json.load(open(os.path.join(golden_dir, "output_sizes.json")))
    for c in g["cases"]:
        assert B.conv_out_dim_dilated(c["in"], c["k"], c["s"], c["p"], 1) == c["out"], c
    assert B.conv_out_dim_dilated(9, 3, 1, 1, 0) == -1
    assert B.conv_out_dim_dilated(9, 3, 1, 1, 1 << 40) == -1


def test_general_validation():
    f = lambda prm, x=X, w=Wp, b=BIAS, y=Y, algo=0: B.conv_fwd_bf16(prm, x, w, b, y, algo, None)
    assert f(None) == 1
    assert f(_gp(), x=None) == 1
    assert f(_gp(), y=None) == 1
    assert f(_gp(dilation=0)) == 2
    assert f(_gp(groups=0)) == 2
    assert f(_gp(groups=3)) == 2                      # does not divide C_in = 8
    assert f(_gp(groups=8, C_out=12)) == 2            # does not divide C_out
    assert f(_gp(ndim=4)) == 2
    assert f(_gp(ndim=1)) == 2
    assert f(_gp(H=6, W=6, pad=0, dilation=3, K=3)) == 3      # span 7 > 6
    assert f(_gp(), algo=9) == 7
    assert f(_gp(), y=X + 64) == 5
    assert B.conv_fwd_f32(_gp(), X, Wp, BIAS, Y, 1, None) == 7        # MFMA is bf16-only
    assert B.conv_fwd_f32(None, X, Wp, BIAS, Y, 0, None) == 1
    assert f(_gp(ndim=3, D=0)) == 2                  # D is read in 3D
    # the weight holds C_out * C_in/groups * K*K elements: y 4 bytes before its end overlaps it
    assert f(_gp(), y=Wp + 16 * 2 * 9 * 2 - 4) == 5


def test_general_xcol_bytes_and_explicit_validation():
    prm = _gp()
    Ho, Wo = B.conv_out_dim_dilated(9, 3, 1, 1, 2), B.conv_out_dim_dilated(11, 3, 1, 1, 2)
    need = 8 * 9 * 2 * Ho * Wo * 2
    assert B.conv_xcol_bytes(prm) == need
    assert B.conv_xcol_bytes(None) == 0
    assert B.conv_xcol_bytes(_gp(groups=3)) == 0
    assert B.conv_xcol_bytes(_gp(ndim=3, D=5)) == 8 * 27 * 2 * B.conv_out_dim_dilated(5, 3, 1, 1, 2) * Ho * Wo * 2
    e = lambda prm, ws=WS, nb=need, y=Y: B.conv_fwd_explicit_bf16(prm, X, Wp, BIAS, y, ws, nb, None)
    assert e(None) == 1
    assert e(prm, ws=None) == 1
    assert e(prm, nb=need - 2) == 6
    assert e(prm, ws=Y + 8) == 5
    assert e(_gp(groups=5)) == 2
    assert B.conv_im2col_bf16(None, X, Y, None) == 1
    assert B.conv_im2col_bf16(prm, None, Y, None) == 1
    assert B.conv_im2col_bf16(prm, X, X + 2, None) == 5
    assert B.conv_im2col_bf16(_gp(dilation=-1), X, Y, None) == 2


def test_backward_validation():
    prm = _gp()                       # (2,8,9,11), (16,2,3,3), s1 p1 d2 G4
    nd, nw = B.conv_bwd_data_workspace_bytes(prm), B.conv_bwd_weight_workspace_bytes(prm)
    # dW workspace: per range of positions, the fp32 partials of dw (C_out x C_in/G x 9) and of db (C_out)
    assert nd >= 16 * 2 * 9 * 2 and nw >= (16 * 2 * 9 + 16) * 4 and nw % ((16 * 2 * 9 + 16) * 4) == 0
    assert B.conv_bwd_data_workspace_bytes(None) == 0 and B.conv_bwd_weight_workspace_bytes(_gp(groups=3)) == 0
    DO = X + 0x01000000
    bd = lambda prm=prm, dout=DO, w=Wp, dx=Y, ws=WS, nb=nd: B.conv_bwd_data_bf16(prm, dout, w, dx, ws, nb, None)
    assert bd(prm=None) == 1 and bd(dout=None) == 1 and bd(dx=None) == 1 and bd(ws=None) == 1
    assert bd(prm=_gp(dilation=0)) == 2
    assert bd(nb=nd - 1) == 6
    assert bd(ws=WS + 8) == 6
    assert bd(dx=DO + 64) == 5            # dx over dout
    assert bd(ws=Y + 64) == 5             # workspace over dx
    bw = lambda prm=prm, x=X, dout=DO, dw=Y, db=BIAS, ws=WS, nb=nw: B.conv_bwd_weight_bf16(prm, x, dout, dw, db, ws, nb, None)
    assert bw(prm=None) == 1 and bw(x=None) == 1 and bw(dout=None) == 1 and bw(dw=None) == 1 and bw(ws=None) == 1
    assert bw(prm=_gp(groups=0)) == 2
    assert bw(nb=nw - 4) == 6
    assert bw(dw=X + 2) == 5              # dw over x
    assert bw(db=DO) == 5                 # db over dout
    assert bw(db=Y + 8) == 5              # db over dw
    assert bw(ws=DO + 32) == 5            # workspace over dout


def test_options_validation():
    prm = _gp()
    f = lambda o, y=Y, algo=0: B.conv_fwd_ex_bf16(prm, o, X, Wp, BIAS, y, None, 0, algo, None)
    assert f(B.ConvOptions(2, 0, 0)) == 2           # unknown layout
    assert f(B.ConvOptions(0, 3, 0)) == 2           # unknown output dtype
    assert f(B.ConvOptions(0, 0, 2)) == 2           # relu not 0/1
    assert B.conv_fwd_ex_bf16(None, None, X, Wp, BIAS, Y, None, 0, 0, None) == 1
    assert B.conv_fwd_ex_f32(prm, B.ConvOptions(0, 0, 0), X, Wp, BIAS, None, 0, None) == 1
    assert B.conv_fwd_ex_f32(prm, B.ConvOptions(1, 1, 1), X, Wp, BIAS, Y, 1, None) == 7   # MFMA is bf16-only
    assert f(B.ConvOptions(0, 1, 0), y=X + 2) == 5   # bf16 output over x
    # 3x3 layers offer the packed-weight workspace with any epilogue and layout
    big = B.make_params((64, 128, 56, 56), (128, 128, 3, 3), 1, 1, 1, 1)
    assert B.conv_fwd_ex_workspace_bytes(big, B.ConvOptions(0, 1, 1), 0) == 128 * 128 * 9 * 2
    assert B.conv_fwd_ex_workspace_bytes(big, None, 0) == 128 * 128 * 9 * 2
    assert B.conv_fwd_ex_workspace_bytes(big, B.ConvOptions(1, 0, 0), 0) == 128 * 128 * 9 * 2   # channels-last too
    assert B.conv_fwd_ex_workspace_bytes(big, B.ConvOptions(0, 0, 5), 0) == 0
    # dilation 2 with pad 2 takes the column-group kernel (packed weights) too; other pads or
    # dilations, and groups, do not
    dil = lambda p, d, g=1: B.make_params((2, 32, 19, 40), (128, 32 // g, 3, 3), 1, p, d, g)
    assert B.conv_fwd_ex_workspace_bytes(dil(2, 2), None, 0) == 128 * 32 * 9 * 2
    assert B.conv_fwd_ex_workspace_bytes(dil(1, 2), None, 0) == 0
    assert B.conv_fwd_ex_workspace_bytes(dil(3, 3), None, 0) == 0
    assert B.conv_fwd_ex_workspace_bytes(dil(2, 2, 2), None, 0) == 0
    # groups of 32 output channels take the grouped column-group kernel (weights packed per group)
    grp = lambda g, co=128, c=128: B.make_params((2, c, 19, 40), (co, c // g, 3, 3), 1, 1, 1, g)
    assert B.conv_fwd_ex_workspace_bytes(grp(4), None, 0) == 128 * 32 * 9 * 2
    assert B.conv_fwd_ex_workspace_bytes(grp(2), None, 0) == 0              # 64 per group: general kernel
    assert B.conv_fwd_ex_workspace_bytes(grp(8, 256, 256), None, 0) == 256 * 32 * 9 * 2
    assert B.conv_fwd_ex_workspace_bytes(grp(4), B.ConvOptions(1, 0, 0), 0) == 0   # channels-last: general
