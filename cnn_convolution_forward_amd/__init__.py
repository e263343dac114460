"""MI355X-native convolution forward engine (conv2d / conv3d, im2col + GEMM).

The compute lives in ``libconvfwd.so`` (hand-written HIP kernels for gfx950 behind
a C ABI declared in ``include/conv_fwd.h``).  ``cnn_convolution_forward_amd.binding``
marshals arguments to it; importing this package does not load the library, but
every compute call does, and raises if it is missing.
"""
__all__ = ["binding", "synth"]
