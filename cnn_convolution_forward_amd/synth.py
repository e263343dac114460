"""Seeded synthetic inputs for the five convolution workloads.

This module is shared by the oracle's tests, the GPU parity tests and the
benchmark.  It holds none of the convolution's arithmetic: it only draws
random tensors and rounds them to the storage type, once, here.

Recipe (the pages fix shapes but not the random generator):
  * ``numpy.random.default_rng(seed)`` (PCG64); draw x, then w, then b, as
    float32; then round x and w to bf16 (round-to-nearest-even) for the bf16
    workloads.  Bias stays fp32.  No NaN or Inf is ever produced.
  * ``N(0, s)`` means standard deviation s = 1/sqrt(fan_in).
  * Integer-valued variants (x, w in {-2..2}, b in {-3..3}) make every partial
    sum an exact small integer, so any correct summation order gives the same
    fp32 bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    ndim: int                      # 2 or 3 spatial dims
    N: int
    C_in: int
    spatial: Tuple[int, ...]       # (H, W) or (D, H, W)
    C_out: int
    K: int
    stride: int
    pad: int
    dtype: str                     # "f32" or "bf16" (input/weight storage)
    x_dist: str                    # "uniform" (U[-1,1]) or "normal" (N(0,1))
    seed: int
    has_bias: bool = True
    dilation: int = 1
    groups: int = 1                # divides C_in and C_out; C_in is depthwise
    note: str = field(default="", compare=False)

    @property
    def plain(self):
        return self.dilation == 1 and self.groups == 1

    @property
    def x_shape(self):
        return (self.N, self.C_in) + tuple(self.spatial)

    @property
    def w_shape(self):
        return (self.C_out, self.C_in // self.groups) + (self.K,) * self.ndim

    @property
    def fan_in(self):
        return self.C_in // self.groups * self.K ** self.ndim

    def out_spatial(self):
        span = self.dilation * (self.K - 1) + 1
        return tuple((d + 2 * self.pad - span) // self.stride + 1 for d in self.spatial)

    @property
    def y_shape(self):
        return (self.N, self.C_out) + self.out_spatial()

    def flops(self) -> int:
        """2 * N * C_out * prod(out) * (C_in/groups) * K^ndim, padded taps included."""
        return 2 * int(np.prod(self.y_shape, dtype=np.int64)) * self.fan_in


# The five workloads, in order: tiny fp32 check, stem, 3x3 (headline), 1x1, conv3d.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 2, 2, 3, (9, 11), 4, 3, 2, 1, "f32", "uniform", 1,
                         note="x (2,3,9,11), w (4,3,3,3), s2 p1 -> (2,4,5,6)"),
    "stem_bf16": Workload("stem_bf16", 2, 32, 3, (224, 224), 64, 3, 2, 1, "bf16", "uniform", 2,
                          note="x (32,3,224,224), w (64,3,3,3), s2 p1 -> (32,64,112,112)"),
    "conv3x3_bf16": Workload("conv3x3_bf16", 2, 64, 128, (56, 56), 128, 3, 1, 1, "bf16", "normal", 3,
                             note="x (64,128,56,56), w (128,128,3,3), s1 p1 -> (64,128,56,56)"),
    "conv1x1_bf16": Workload("conv1x1_bf16", 2, 32, 256, (28, 28), 1024, 1, 1, 0, "bf16", "normal", 4,
                             note="x (32,256,28,28), w (1024,256,1,1) -> (32,1024,28,28)"),
    "conv3d_bf16": Workload("conv3d_bf16", 3, 8, 3, (16, 64, 64), 64, 3, 1, 1, "bf16", "uniform", 5,
                            note="x (8,3,16,64,64), w (64,3,3,3,3), s1 p1 -> (8,64,16,64,64)"),
}
HEADLINE = "conv3x3_bf16"

# Dilation and groups at the 3x3 layer's size (64 x 128 x 56 x 56, N(0,1) inputs,
# N(0, 1/sqrt(fan_in)) weights): depthwise (groups = C_in, weight (128,1,3,3)),
# dilation 2 with pad 2 (size kept), and groups = 4 (weight (128,32,3,3)).
WORKLOADS_GENERAL = {
    "depthwise3x3_bf16": Workload("depthwise3x3_bf16", 2, 64, 128, (56, 56), 128, 3, 1, 1, "bf16", "normal", 6,
                                  groups=128, note="x (64,128,56,56), w (128,1,3,3), groups 128 -> (64,128,56,56)"),
    "dilated3x3_bf16": Workload("dilated3x3_bf16", 2, 64, 128, (56, 56), 128, 3, 1, 2, "bf16", "normal", 7,
                                dilation=2, note="x (64,128,56,56), w (128,128,3,3), d2 p2 -> (64,128,56,56)"),
    "grouped3x3_bf16": Workload("grouped3x3_bf16", 2, 64, 128, (56, 56), 128, 3, 1, 1, "bf16", "normal", 8,
                                groups=4, note="x (64,128,56,56), w (128,32,3,3), groups 4 -> (64,128,56,56)"),
}
# The 3x3 layer at one GPU's share of an 8-way batch shard (N = 8): the same
# per-image work, 112 tiles of the column-group kernel for 256 compute units.
WORKLOADS_SHARD = {
    "conv3x3_bf16_n8": Workload("conv3x3_bf16_n8", 2, 8, 128, (56, 56), 128, 3, 1, 1, "bf16", "normal", 9,
                                note="x (8,128,56,56), w (128,128,3,3), s1 p1 -> (8,128,56,56)"),
}
ALL_WORKLOADS = {**WORKLOADS, **WORKLOADS_GENERAL, **WORKLOADS_SHARD}


@dataclass
class Tensors:
    x: np.ndarray                 # uint16 bf16 bits, or float32
    w: np.ndarray
    b: Optional[np.ndarray]       # float32 or None
    seed: int


def make_inputs(wl: Workload, seed: Optional[int] = None, integer: bool = False,
                with_bias: Optional[bool] = None, shape_override=None) -> Tensors:
    """Draw x, w, b for ``wl`` (optionally at another shape: a dict of fields).

    Storage: bf16 workloads return x and w as uint16 bit patterns, fp32
    workloads as float32; bias is float32 or None.
    """
    if shape_override:
        wl = Workload(**{**wl.__dict__, **shape_override})
    seed = wl.seed if seed is None else seed
    with_bias = wl.has_bias if with_bias is None else with_bias
    rng = np.random.default_rng(seed)
    if integer:
        x = rng.integers(-2, 3, size=wl.x_shape).astype(np.float32)
        w = rng.integers(-2, 3, size=wl.w_shape).astype(np.float32)
        b = rng.integers(-3, 4, size=(wl.C_out,)).astype(np.float32)
    else:
        if wl.x_dist == "uniform":
            x = rng.uniform(-1.0, 1.0, size=wl.x_shape).astype(np.float32)
        else:
            x = rng.standard_normal(size=wl.x_shape, dtype=np.float32)
        if wl.dtype == "f32":
            w = rng.uniform(-1.0, 1.0, size=wl.w_shape).astype(np.float32)
        else:
            sigma = np.float32(1.0 / np.sqrt(wl.fan_in))
            w = (rng.standard_normal(size=wl.w_shape, dtype=np.float32) * sigma).astype(np.float32)
        b = rng.uniform(-1.0, 1.0, size=(wl.C_out,)).astype(np.float32)
    if wl.dtype == "bf16":
        x, w = f32_to_bf16_bits(x), f32_to_bf16_bits(w)
    return Tensors(x=x, w=w, b=b if with_bias else None, seed=seed)


def workload(name: str, **override) -> Workload:
    wl = ALL_WORKLOADS[name]
    return Workload(**{**wl.__dict__, **override}) if override else wl
