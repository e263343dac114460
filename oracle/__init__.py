"""CPU oracle for the convolution forward pass (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .oracle import (build, col2im_dilated, conv2d, conv3d, conv_backward, conv_backward_points,  # noqa: F401
                     conv_general, conv_general_points, conv_nhwc, conv_points, decode, epilogue,
                     im2col2d, im2col3d, im2col_dilated, matmul, num_threads, out_dim, out_dim_dilated,
                     round_bf16, winograd_f2x2_3x3)
