"""Planted mistakes in a copy of the oracle must fail the pins.

Each case edits one line of a temporary copy of oracle/conv_ref.c (a plausible
slip: sign of the padding offset, kh/kw swapped, bias dropped, X_col columns
transposed, a depth offset lost, |x*w| replaced by x*w, ceil for floor, an
off-by-one bounds check; in the dilation/groups functions: dilation dropped
from an axis, groups interleaved, the group's channel offset lost, the dilated
span mis-sized; in the backward pass: dx overwritten, dW from w, db over one
image, the stride or group offset lost, col2im overwriting; in the epilogue:
bf16 ties rounded away or truncated, ReLU keeping negatives, the channels-last
group offset lost; in Winograd: a transform sign or coefficient, the output
rows, the block origin), builds it with gcc, and runs the matching pin file
(tests/test_oracle_pins*.py) against that build in a subprocess.  The run must fail.  Runs on the CPU only.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "conv_ref.c")

MUTANTS = {
    "pad_sign": ("int64_t ih = oh * s + kh - p;", "int64_t ih = oh * s + kh + p;"),
    "kh_kw_swapped": ("double wv = w[(((oc * C + ic) * Kd + kd) * K + kh) * K + kw];",
                      "double wv = w[(((oc * C + ic) * Kd + kd) * K + kw) * K + kh];"),
    "bias_dropped": ("y[o] = acc + (bias ? bias[oc] : 0.0);\n                    if (S) S[o] = sa;\n                }\n    return 0;\n}\n\n/* Full 3D",
                     "y[o] = acc;\n                    if (S) S[o] = sa;\n                }\n    return 0;\n}\n\n/* Full 3D"),
    "xcol_columns_transposed": ("col[r * cols + (n * Ho + oh) * Wo + ow] = v;",
                                "col[r * cols + (n * Wo + ow) * Ho + oh] = v;"),
    "depth_pad_lost": ("int64_t id = od * sd + kd - pd;", "int64_t id = od * sd + kd;"),
    "S_signed": ("S += fabs(t);", "S += t;"),
    "ceil_size": ("return num / s + 1;", "return (num + s - 1) / s + 1;"),
    "lower_bound_strict": ("if (!(0 <= ih && ih < H)) continue;", "if (!(0 < ih && ih < H)) continue;"),
    "stride_dropped_w": ("int64_t iw = ow * s + kw - p;\n                    if (!(0 <= iw",
                         "int64_t iw = ow + kw - p;\n                    if (!(0 <= iw"),
}

# Mistakes in the dilation / groups functions, caught by test_oracle_pins_general.py.
MUTANTS_GENERAL = {
    "dilation_dropped_h": ("const int64_t iy = oh * g->s + kh * g->d - g->p;",
                           "const int64_t iy = oh * g->s + kh - g->p;"),
    "depth_dilation_dropped": ("const int64_t iz = od * g->sz + kz * g->dz - g->pz;",
                               "const int64_t iz = od * g->sz + kz - g->pz;"),
    "groups_interleaved": ("const int64_t grp = oc / Cog;\n    double acc", "const int64_t grp = oc % g->G;\n    double acc"),
    "group_offset_dropped": ("const int64_t ic = grp * Cg + j;\n        for (int64_t kz = 0; kz < g->Kz; ++kz) {",
                             "const int64_t ic = j + 0 * grp;\n        for (int64_t kz = 0; kz < g->Kz; ++kz) {"),
    "dilated_span_wrong": ("int64_t span = d * (k - 1) + 1;", "int64_t span = d * k - d + 1 + (d > 1);"),
    "im2col_dilation_dropped_w": ("const int64_t iy = oh * s + kh * d - p, ix = ow * s + kw * d - p;\n                double v",
                                  "const int64_t iy = oh * s + kh * d - p, ix = ow * s + kw - p;\n                double v"),
}


# Mistakes in the backward pass and col2im, caught by test_oracle_pins_backward.py.
MUTANTS_BACKWARD = {
    "dx_overwritten": ("if (dx) dx[xi] += w[wi] * gout;", "if (dx) dx[xi] = w[wi] * gout;"),
    "dw_from_w": ("if (dw) dw[wi] += gout * x[xi];", "if (dw) dw[wi] += gout * w[wi];"),
    "db_one_image": ("if (db) db[oc] += gout;", "if (db && n == 0) db[oc] += gout;"),
    "bwd_stride_dropped": ("                    const int64_t iy = oh * s + kh * d - p;\n",
                           "                    const int64_t iy = oh + kh * d - p;\n"),
    "bwd_group_offset_dropped": ("const int64_t ic = grp * Cg + j;\n                for (int64_t kz = 0; kz < g.Kz; ++kz) {",
                                 "const int64_t ic = j + 0 * grp;\n                for (int64_t kz = 0; kz < g.Kz; ++kz) {"),
    "col2im_overwrites": ("dx[(((n * C + ic) * g.Dd + iz) * H + iy) * W + ix] += col[r * cols + n * plane + q];",
                          "dx[(((n * C + ic) * g.Dd + iz) * H + iy) * W + ix] = col[r * cols + n * plane + q];"),
}

# Mistakes in the epilogue and the channels-last convolution, caught by test_oracle_pins_epilogue.py.
MUTANTS_EPILOGUE = {
    "bf16_ties_away": ("if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;",
                       "if (frac >= 0.5) r += 1.0;"),
    "bf16_truncates": ("if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;",
                       "if (frac > 2.0) r += 1.0;"),
    "relu_keeps_negatives": ("if (relu && v < 0.0) v = 0.0;", "if (relu && v < -1e300) v = 0.0;"),
    "nhwc_group_offset_dropped": ("* W + ix) * C + grp * Cg;", "* W + ix) * C + 0 * grp * Cg;"),
}

# Mistakes in Winograd F(2x2,3x3), caught by test_oracle_pins_winograd.py.
MUTANTS_WINOGRAD = {
    "wino_bt_sign": ("static const double BT[4][4] = {{1, 0, -1, 0}, {0, 1, 1, 0}, {0, -1, 1, 0}, {0, 1, 0, -1}};",
                     "static const double BT[4][4] = {{1, 0, 1, 0}, {0, 1, 1, 0}, {0, -1, 1, 0}, {0, 1, 0, -1}};"),
    "wino_g_coefficient": ("{0.5, -0.5, 0.5}, {0, 0, 1}};", "{0.5, -0.5, 1.0}, {0, 0, 1}};"),
    "wino_at_rows_swapped": ("static const double AT[2][4] = {{1, 1, 1, 0}, {0, 1, -1, -1}};",
                             "static const double AT[2][4] = {{0, 1, -1, -1}, {1, 1, 1, 0}};"),
    "wino_block_origin": ("const int64_t ih = 2 * bh - p + i, iw = 2 * bw - p + j;",
                          "const int64_t ih = 2 * bh - p + i, iw = 2 * bw + j;"),
}

CASES = [(n, "test_oracle_pins.py") for n in sorted(MUTANTS)] + \
        [(n, "test_oracle_pins_general.py") for n in sorted(MUTANTS_GENERAL)] + \
        [(n, "test_oracle_pins_backward.py") for n in sorted(MUTANTS_BACKWARD)] + \
        [(n, "test_oracle_pins_epilogue.py") for n in sorted(MUTANTS_EPILOGUE)] + \
        [(n, "test_oracle_pins_winograd.py") for n in sorted(MUTANTS_WINOGRAD)]


@pytest.mark.parametrize("name,pins", CASES)
def test_planted_mistake_is_caught(name, pins, tmp_path):
    old, new = {**MUTANTS, **MUTANTS_GENERAL, **MUTANTS_BACKWARD, **MUTANTS_EPILOGUE, **MUTANTS_WINOGRAD}[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found once: %s" % name
    mutant_c = tmp_path / "conv_ref_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           "-o", str(so), str(mutant_c), "-lm"])
    env = dict(os.environ, CONV_ORACLE_LIB_OVERRIDE=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "planted mistake %r passed every pin:\n%s" % (name, r.stdout[-2000:])
