"""CPU oracle for the convolution forward pass (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .oracle import (build, conv2d, conv3d, conv_points, decode, im2col2d, im2col3d,  # noqa: F401
                     matmul, num_threads, out_dim)
