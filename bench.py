#!/usr/bin/env python3
"""Benchmark: convolution forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--route auto|mfma|valu|explicit]
                    [--no-cpu-baseline] [--report]

A step is one full forward pass of the convolution (every kernel of the chosen
route, the weight repack included) over one batch of seeded synthetic input
that is already resident in device memory.  W untimed steps, then exactly K
timed steps bracketed by torch.cuda.synchronize().  The default workload is
the 3x3 layer (N=64, C_in=C_out=128, 56x56, stride 1, pad 1, bf16 in, fp32
out).

One JSON line on stdout:
  value        FLOP/s of the whole job (2*N*C_out*H_out*W_out*C_in*K^2, padded
               taps included) / measured time, in TFLOP/s
  roofline     the dominant kernel (the convolution): algorithmic FLOP (or
               bytes) per launch over its average launch time from HIP events
               recorded on the stream the library launches on, against the
               MI355X peak; traffic = HBM bytes per launch from rocprofv3
               counters (profiles/counters_*.json) while they match the
               current kernel sources, else null
  cpu_baseline the CPU oracle (plain fp64 loops, OpenMP) timed on the same
               inputs on this host (the whole batch unless told otherwise)
--report prints one more line per workload to stderr (every workload, every route).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "conv fwd TFLOP/s + % bf16 MFMA peak (3x3 s1p1, N=64 C=128 56x56)"
PEAK_BF16_TFLOPS = 2516.6          # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP32_VALU_TFLOPS = 157.3      # packed; 78.6 without packed FMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps before the timed ones (after the clock-settling phase)")
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="before the warm-up steps, run whole steps untimed until this much GPU time has passed: "
                         "an idle GPU starts at a low clock and reaches its loaded clock after ~40 ms of "
                         "continuous work (reported as clock_settle; 0 disables)")
    ap.add_argument("--workload", default="conv3x3_bf16")
    ap.add_argument("--route", default="auto", choices=["auto", "mfma", "valu", "explicit", "winograd", "plain"],
                    help="plain: the 2D entry point without a workspace (conv2d_fwd_bf16), AUTO's kernel choice")
    ap.add_argument("--layout", default="nchw", choices=["nchw", "nhwc"], help="layout of x and y (forward)")
    ap.add_argument("--out", default="f32", choices=["f32", "bf16"], help="output dtype (forward)")
    ap.add_argument("--relu", action="store_true", help="fused ReLU after the bias (forward)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass instead (data + weight + bias gradients of the layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache pass (50 steps, caches evicted "
                                                            "before each)")
    ap.add_argument("--cpu-sample-images", type=int, default=0,
                    help="images in the oracle's timed sample (0 = the whole batch)")
    ap.add_argument("--report", action="store_true", help="also time every workload/route (stderr)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only time plain streaming kernels (torch's fill, bf16 -> fp32 conversion, copy and sum, "
                         "and hipMemsetAsync) at the 3x3 layer's byte counts: the HBM rates a plain kernel reaches "
                         "on this chip, beside the 8 TB/s peak")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times): the "
                         "reference dispatch for scaling HBM byte counters")
    return ap.parse_args()


def algorithmic_bytes(wl, out_bytes=4):
    """x, w, bias read once + y written once (fp32 output, or bf16 with out_bytes=2)."""
    esz = 4 if wl.dtype == "f32" else 2
    x = int(np.prod(wl.x_shape)) * esz
    w = int(np.prod(wl.w_shape)) * esz
    b = wl.C_out * 4
    y = int(np.prod(wl.y_shape)) * out_bytes
    return x + w + b + y


def xcol_bytes(wl):
    """Bytes of the explicit route's patch matrix X_col (C_in*K^dims rows x
    N*prod(out) columns, bf16)."""
    rows = wl.C_in * wl.K ** wl.ndim          # every group's rows: C_in * K^dims whatever the groups
    cols = wl.N * int(np.prod(wl.out_spatial()))
    return rows * cols * 2


def route_bytes(wl, route, out_bytes=4):
    """Algorithmic bytes of one forward call on `route`: the implicit routes
    read x, w, bias once and write y once; the explicit route also writes
    X_col and reads it back (x + 2*X_col + w + bias + y)."""
    ab = algorithmic_bytes(wl, out_bytes)
    return ab + 2 * xcol_bytes(wl) if route == "explicit" else ab


def bound_of(wl, route, out_bytes=4):
    if route == "explicit":
        return "hbm"                  # X_col written and read back: ~55 FLOP/byte on the 3x3 layer
    ab = algorithmic_bytes(wl, out_bytes)
    if wl.dtype == "f32" or route == "valu":
        return "alu" if wl.flops() / ab > PEAK_FP32_VALU_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    return "mfma" if wl.flops() / ab > ridge else "hbm"


class Runner:
    """Device-resident inputs and one callable step for a workload/route.

    A step is everything one forward pass needs: for the 2D bf16 MFMA route
    with packed weights, the weight repack (conv2d_pack_weights_bf16) and the
    convolution (conv2d_fwd_bf16_prepacked); otherwise the one library call.
    `main()` is the launch whose duration the roofline uses (the convolution)."""

    def __init__(self, wl, route, seed=None, backward=False, options=None):
        import torch
        from cnn_convolution_forward_amd import binding as B
        from cnn_convolution_forward_amd import synth
        self.wl, self.route, self.backward = wl, route, backward
        # (layout, out dtype, relu); None = NCHW, fp32, no ReLU
        self.options = None if options in (None, ("nchw", "f32", False)) else options
        if route == "winograd" and self.options is None:
            self.options = ("nchw", "f32", False)       # Winograd runs through the options entry point
        if (self.options is None and not backward and not wl.plain and wl.dtype == "bf16" and
                route in ("auto", "mfma")):
            # dilation / groups: the workspace entry point (with its packed 3x3
            # weights the column-group kernel takes dilation 1 or 2)
            self.options = ("nchw", "f32", False)
        self.t = synth.make_inputs(wl, seed=seed)
        t = self.t
        if t.x.dtype == np.uint16:
            self.x = torch.from_numpy(t.x.view(np.int16)).cuda()
            self.w = torch.from_numpy(t.w.view(np.int16)).cuda()
        else:
            self.x = torch.from_numpy(t.x).cuda()
            self.w = torch.from_numpy(t.w).cuda()
        self.b = None if t.b is None else torch.from_numpy(t.b).cuda()
        self.y = torch.empty(wl.y_shape, dtype=torch.float32, device="cuda")
        if self.options is not None:
            layout, out, relu = self.options
            if layout == "nhwc":
                # the same values, stored channels-last
                perm = (0,) + tuple(range(2, wl.ndim + 2)) + (1,)
                self.x = self.x.permute(*perm).contiguous()
                yshape = (wl.y_shape[0],) + tuple(wl.y_shape[2:]) + (wl.y_shape[1],)
            else:
                yshape = wl.y_shape
            self.y = torch.empty(yshape, dtype=torch.int16 if out == "bf16" else torch.float32, device="cuda")
            self.opts = B.ConvOptions(B.LAYOUT[layout], B.OUT_DTYPE[out], int(bool(relu)))
        self.ws = None
        self.packed = None
        # dilation / groups go through the general entry points (conv_params_t)
        self.params = None if wl.plain else B.make_params(wl.x_shape, wl.w_shape, wl.stride, wl.pad,
                                                          wl.dilation, wl.groups)
        if self.options is not None:
            self.params = B.make_params(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups)
            n = B.conv_fwd_ex_workspace_bytes(self.params, self.opts, B.ALGO.get(route, 0))
            self.ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
        elif route in ("auto", "mfma") and wl.ndim == 2 and wl.dtype == "bf16" and wl.plain:
            self.packed = B.workspace_for(self.x, self.w, wl.stride, wl.pad, route)
        # route "plain": no workspace, no packed weights: the one conv2d_fwd_bf16 call
        if route == "explicit":
            if self.params is not None:
                nbytes = B.conv_xcol_bytes(self.params)
            else:
                nbytes = B.conv_im2col_bytes(wl.ndim, wl.N, wl.C_in, wl.spatial[0] if wl.ndim == 3 else 1,
                                             wl.spatial[-2], wl.spatial[-1], wl.K, wl.stride, wl.pad)
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        if backward:
            # upstream gradient: N(0,1), bf16, from the workload seed + 1000
            rng = np.random.default_rng(wl.seed + 1000)
            self.dout_np = synth.f32_to_bf16_bits(rng.standard_normal(size=wl.y_shape, dtype=np.float32))
            self.dout = torch.from_numpy(self.dout_np.view(np.int16)).cuda()
            self.dx = torch.empty(wl.x_shape, dtype=torch.float32, device="cuda")
            self.dw = torch.empty(wl.w_shape, dtype=torch.float32, device="cuda")
            self.db = torch.empty((wl.C_out,), dtype=torch.float32, device="cuda")
            self.params = B.make_params(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups)
            self.wsd = torch.empty(max(16, B.conv_bwd_data_workspace_bytes(self.params)), dtype=torch.uint8,
                                   device="cuda")
            self.wsw = torch.empty(max(16, B.conv_bwd_weight_workspace_bytes(self.params)), dtype=torch.uint8,
                                   device="cuda")
        self.B = B
        self._bind()

    def _bind(self):
        """Resolve every argument of the library calls once (device pointers,
        sizes, the stream), so a step is one or two plain C calls."""
        import torch
        B, wl = self.B, self.wl
        L = B.lib()
        st = torch.cuda.current_stream().cuda_stream
        ptr = lambda t: None if t is None else t.data_ptr()
        sp = list(wl.spatial)
        D = sp[0] if wl.ndim == 3 else 1
        H, W = sp[-2], sp[-1]
        algo = B.ALGO.get(self.route, 0)
        x, w, b, y = ptr(self.x), ptr(self.w), ptr(self.b), ptr(self.y)
        self._pre = None
        self._im2col = None
        if self.options is not None:
            prm, opt = ctypes.byref(self.params), ctypes.byref(self.opts)
            if wl.dtype == "f32":
                self._main = (L.conv_fwd_ex_f32, (prm, opt, x, w, b, y, algo, st))
            else:
                nb = 0 if self.ws is None else self.ws.numel()
                self._main = (L.conv_fwd_ex_bf16, (prm, opt, x, w, b, y, ptr(self.ws), nb, algo, st))
        elif self.backward:
            prm = ctypes.byref(self.params)
            self._pre = (L.conv_bwd_data_bf16, (prm, ptr(self.dout), w, ptr(self.dx), ptr(self.wsd),
                                                self.wsd.numel(), st))
            self._main = (L.conv_bwd_weight_bf16, (prm, x, ptr(self.dout), ptr(self.dw), ptr(self.db),
                                                   ptr(self.wsw), self.wsw.numel(), st))
        elif self.params is not None:
            prm = ctypes.byref(self.params)
            if self.route == "explicit":
                self._main = (L.conv_fwd_explicit_bf16, (prm, x, w, b, y, ptr(self.ws), self.ws.numel(), st))
            else:
                fn = L.conv_fwd_f32 if wl.dtype == "f32" else L.conv_fwd_bf16
                self._main = (fn, (prm, x, w, b, y, algo, st))
        elif self.route == "explicit":
            nb = self.ws.numel()
            if wl.ndim == 2:
                self._im2col = (L.conv2d_im2col_bf16, (x, ptr(self.ws), wl.N, wl.C_in, H, W, wl.K, wl.stride,
                                                       wl.pad, st))
            else:
                self._im2col = (L.conv3d_im2col_bf16, (x, ptr(self.ws), wl.N, wl.C_in, D, H, W, wl.K, wl.stride,
                                                       wl.pad, st))
            if wl.ndim == 2:
                self._main = (L.conv2d_fwd_bf16_explicit,
                              (x, w, b, y, ptr(self.ws), nb, wl.N, wl.C_in, H, W, wl.C_out, wl.K, wl.stride, wl.pad, st))
            else:
                self._main = (L.conv3d_fwd_bf16_explicit,
                              (x, w, b, y, ptr(self.ws), nb, wl.N, wl.C_in, D, H, W, wl.C_out, wl.K, wl.stride,
                               wl.pad, st))
        elif self.packed is not None:
            nb = self.packed.numel()
            dims = (wl.N, wl.C_in, H, W, wl.C_out, wl.K, wl.stride, wl.pad, algo, st)
            self._pre = (L.conv2d_pack_weights_bf16, (w, ptr(self.packed), nb) + dims)
            self._main = (L.conv2d_fwd_bf16_prepacked, (x, ptr(self.packed), nb, b, y) + dims)
        else:
            f32 = wl.dtype == "f32"
            if wl.ndim == 2:
                fn = L.conv2d_fwd_f32 if f32 else L.conv2d_fwd_bf16
                args = (x, w, b, y, wl.N, wl.C_in, H, W, wl.C_out, wl.K, wl.stride, wl.pad, algo, st)
            else:
                fn = L.conv3d_fwd_f32 if f32 else L.conv3d_fwd_bf16
                args = (x, w, b, y, wl.N, wl.C_in, D, H, W, wl.C_out, wl.K, wl.stride, wl.pad, algo, st)
            self._main = (fn, args)

    def _call(self, fa):
        rc = fa[0](*fa[1])
        if rc != 0:
            raise self.B.ConvError(rc, fa[0].__name__)

    def pre(self):
        """Work of the step that precedes the measured launch (weight repack)."""
        if self._pre is not None:
            self._call(self._pre)

    def main(self):
        self._call(self._main)

    def step(self):
        self.pre()
        self.main()

    def im2col(self):
        """The explicit route's first kernel alone (X_col written to the workspace)."""
        self._call(self._im2col)


def _batched(fn, steps, batches=5):
    """GPU time per call of `fn` run `steps` times back to back, in `batches`
    equal runs each bracketed by one pair of HIP events on the current stream
    (the one the library launches on): no event packet between two calls.
    Returns (mean, median of the batch means, min of the batch means), seconds."""
    import torch
    stream = torch.cuda.current_stream()
    per = max(1, steps // batches)
    means = []
    for _ in range(batches):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(per):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        means.append(a.elapsed_time(b) * 1e-3 / per)
    return float(np.mean(means)), float(np.median(means)), float(np.min(means))


def settle_clock(runner, ms):
    """Run whole steps, untimed, in chunks of 16 until `ms` of GPU time has
    passed (HIP events around each chunk); returns (steps run, GPU ms)."""
    import torch
    if ms <= 0:
        return 0, 0.0
    stream = torch.cuda.current_stream()
    n, total = 0, 0.0
    while total < ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(16):
            runner.step()
        b.record(stream)
        torch.cuda.synchronize()
        total += a.elapsed_time(b)
        n += 16
    return n, total


def time_steps(runner, steps, warmup, settle_ms=0.0):
    """After the clock-settling phase (settle_clock) and `warmup` untimed steps:

    A. exactly `steps` steps back to back, bracketed by synchronize (the wall
       clock, for `value`) and by one pair of HIP events (GPU time);
    then, for the roofline, the measured launch alone (`runner.main`, e.g. the
    convolution with weights already packed) `steps` times back to back, and
    the step's other work (`runner.pre`, the weight repack) alone likewise,
    each in batches bracketed by one event pair (no events between launches,
    so the launch time cannot exceed the step's).
    """
    import torch
    runner.settle = settle_clock(runner, settle_ms)
    for _ in range(warmup):
        runner.step()
    stream = torch.cuda.current_stream()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for _ in range(steps):
        runner.step()
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu = g0.elapsed_time(g1) * 1e-3
    main = _batched(runner.main, steps)
    pre = _batched(runner.pre, steps) if runner._pre is not None else (0.0, 0.0, 0.0)
    runner.pre_per = pre
    return wall, gpu, main


def time_cold(runner, steps, flush_bytes=512 << 20):
    """Cold caches: before each step a reduction reads `flush_bytes` of a scratch
    buffer (outside the events), which evicts the L2s and the 256 MB memory-side
    cache and leaves them holding clean lines (a write would leave dirty lines
    for the step to write back); events around the step and its measured
    launch."""
    import torch
    stream = torch.cuda.current_stream()
    scratch = torch.ones(flush_bytes // 4, dtype=torch.int32, device="cuda")
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    for i in range(steps):
        scratch.max()
        a, b, c = ev[i]
        a.record(stream)
        runner.pre()
        b.record(stream)
        runner.main()
        c.record(stream)
    torch.cuda.synchronize()
    step = np.array([a.elapsed_time(c) for a, _, c in ev]) * 1e-3
    main = np.array([b.elapsed_time(c) for _, b, c in ev]) * 1e-3
    del scratch
    return step, main


# HBM traffic of the main kernel from rocprofv3 counters (profiles/counters_*.json):
# FETCH_SIZE and WRITE_SIZE per dispatch, scaled by what they read for a plain
# copy of known size.  Used only while the kernel sources still hash to the
# value recorded with the counters.
def kernel_sources_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counters_from_profiles(workload, route):
    """The committed counter summary for (workload, route), while the kernel
    sources still hash to the value recorded with it: a dict with
    hbm_bytes_per_dispatch and, where recorded, mfma_busy (SQ_VALU_MFMA_BUSY_CYCLES
    over the SIMD cycles of the dispatch) and sclk_mhz (GRBM_GUI_ACTIVE cycles
    over the dispatch duration)."""
    import glob
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "counters_*.json"))):
        with open(f) as fh:
            c = json.load(fh)
        if c.get("workload") != workload or c.get("route") != route:
            continue
        if kernel_sources_sha(c["sources"]) != c["sources_sha256"]:
            return None, "counters in %s predate the current kernel sources" % os.path.basename(f)
        return c, os.path.basename(f)
    return None, "no counter summary for this workload"


def roofline_entry(wl, route, kernel_s, out_bytes=4, counters=None):
    """The roofline object of the dominant launch: algorithmic FLOP (MFMA or
    ALU bound) or bytes (HBM bound) per launch over its time, against the
    MI355X peak of that resource."""
    bound = bound_of(wl, route, out_bytes)
    if bound == "mfma":
        ach, peak, unit = wl.flops() / kernel_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    elif bound == "alu":
        ach, peak, unit = wl.flops() / kernel_s / 1e12, PEAK_FP32_VALU_TFLOPS, "TFLOP/s"
    else:
        ach, peak, unit = route_bytes(wl, route, out_bytes) / kernel_s / 1e9, PEAK_HBM_GBS, "GB/s"
    r = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
         "traffic": None, "algorithmic": wl.flops() if bound in ("mfma", "alu") else route_bytes(wl, route, out_bytes)}
    if counters:
        r["traffic"] = counters.get("hbm_bytes_per_dispatch")
        for k in ("mfma_busy", "sclk_mhz"):
            if k in counters:
                r[k] = counters[k]
        if "sclk_mhz" in counters and bound == "mfma":
            # the same fraction against the peak at the clock the counters measured
            r["frac_at_measured_sclk"] = round(ach / (peak * counters["sclk_mhz"] / 2400.0), 4)
    return r


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, runner, sample_images):
    """Time the oracle on the first `sample_images` images of the same inputs
    (the whole batch by default); also report the parity of the GPU output on
    that sample."""
    import oracle
    t = runner.t
    n = sample_images
    xs = t.x[:n]
    layout, out, relu = runner.options or ("nchw", "f32", False)
    t0 = time.perf_counter()
    if wl.plain and runner.options is None:
        f = oracle.conv2d if wl.ndim == 2 else oracle.conv3d
        y_ref, S = f(xs, t.w, t.b, wl.stride, wl.pad)
    else:
        y_ref, S = oracle.conv_general(xs, t.w, t.b, wl.stride, wl.pad, wl.dilation, wl.groups)
        if relu or out == "bf16":
            y_ref = oracle.epilogue(y_ref, relu=relu)
    dt = time.perf_counter() - t0
    flops = wl.flops() * n / wl.N
    y_gpu = runner.y[:n].cpu()
    if out == "bf16":
        from cnn_convolution_forward_amd import synth
        y_gpu = synth.bf16_bits_to_f32(y_gpu.numpy().view(np.uint16))
    else:
        y_gpu = y_gpu.numpy()
    if layout == "nhwc":
        y_gpu = np.moveaxis(y_gpu, -1, 1)
    y_gpu = y_gpu.astype(np.float64)
    d = np.abs(y_gpu - y_ref)
    tau = 1e-3 if wl.dtype == "bf16" else 1e-5
    ok = bool(np.all(d <= tau * S + (2.0 ** -8 * np.abs(y_ref) if out == "bf16" else 0.0)))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = float(np.max(np.where(S > 0, d / np.where(S > 0, S, 1), 0.0)))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": "%d of %d images of the same seeded inputs (one full forward pass over them), "
                      "fp64" % (n, wl.N),
            "parity_on_sample": {"max_abs_delta_over_S": rel, "tau": tau, "pass": ok}}


def cpu_baseline_backward(wl, runner, sample_images):
    """The oracle's backward loop on the first `sample_images` images (with
    their dout); parity of the GPU dx on those images (dx of an image depends
    on that image's dout only)."""
    import oracle
    n = sample_images
    t = runner.t
    t0 = time.perf_counter()
    (dx, _, _), (Sdx, _, _) = oracle.conv_backward(t.x[:n], t.w, runner.dout_np[:n], wl.stride, wl.pad,
                                                   wl.dilation, wl.groups)
    dt = time.perf_counter() - t0
    flops = 2 * wl.flops() * n / wl.N
    g = runner.dx[:n].cpu().numpy().astype(np.float64)
    d = np.abs(g - dx)
    ok = bool(np.all(d <= 1e-3 * Sdx))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = float(np.max(np.where(Sdx > 0, d / np.where(Sdx > 0, Sdx, 1), 0.0)))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "cpu_model": cpu_model(), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": "%d of %d images of the same seeded inputs and upstream gradient (dx, dW and db over "
                      "them, the scatter loop, one thread), fp64" % (n, wl.N),
            "parity_on_sample": {"dx_max_abs_delta_over_S": rel, "tau": 1e-3, "pass": ok}}


def describe(wl):
    extra = {} if wl.plain else {"dilation": wl.dilation, "groups": wl.groups}
    return {"workload": wl.name, "x": list(wl.x_shape), "w": list(wl.w_shape), "y": list(wl.y_shape),
            "stride": wl.stride, "pad": wl.pad, **extra, "in_dtype": wl.dtype, "out_dtype": "f32",
            "seed": wl.seed, "flop_per_step": wl.flops(), "algorithmic_bytes_per_step": algorithmic_bytes(wl)}


def measure(wl, route, steps, warmup, backward=False, options=None, settle_ms=0.0):
    runner = Runner(wl, route, backward=backward, options=options)
    wall, gpu, per = time_steps(runner, steps, warmup, settle_ms)
    return runner, wall, gpu, per


def report_all(steps, warmup):
    from cnn_convolution_forward_amd import synth
    for name, wl in synth.ALL_WORKLOADS.items():
        routes = ["valu"] if wl.dtype == "f32" else ["auto", "mfma", "valu", "explicit"] + (["plain"] if wl.plain and wl.ndim == 2 else [])
        for route in routes:
            _, wall, gpu, per = measure(wl, route, steps, warmup)
            t = per[0]
            line = {"workload": name, "route": route, "us_per_call": round(t * 1e6, 2),
                    "us_per_step": round(wall / steps * 1e6, 2),
                    "TFLOP/s": round(wl.flops() / t / 1e12, 2),
                    "pct_bf16_mfma_peak": round(100 * wl.flops() / t / 1e12 / PEAK_BF16_TFLOPS, 2),
                    "algorithmic_GB/s": round(algorithmic_bytes(wl) / t / 1e9, 1),
                    "pct_hbm_peak": round(100 * algorithmic_bytes(wl) / t / 1e9 / PEAK_HBM_GBS, 2)}
            print(json.dumps(line), file=sys.stderr, flush=True)


def stream_probe(reps=50):
    """HBM rates of plain streaming kernels on the 3x3 layer's buffers: x is
    51.4 MB of bf16, y 102.8 MB of fp32.  Each op runs `reps` times back to
    back between one pair of HIP events, after 20 untimed runs; one JSON line
    per op with its bytes moved and TB/s."""
    import torch
    stream = torch.cuda.current_stream()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemsetAsync.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p]
    ops = []
    # the 3x3 layer's sizes (x and y together fit the 256 MB memory-side
    # cache, as in back-to-back launches of the layer), then 8x larger
    # buffers that do not
    for scale, tag in ((1, "3x3-layer size"), (8, "8x the 3x3 layer")):
        n_x = 64 * 128 * 56 * 56 * scale
        xb = torch.ones(n_x, dtype=torch.bfloat16, device="cuda")
        y = torch.empty(n_x, dtype=torch.float32, device="cuda")
        y2 = torch.empty_like(y)
        ops += [
            ("fill fp32 y (write only), " + tag, lambda y=y: y.fill_(1.0), 4 * n_x),
            ("hipMemsetAsync y (write only), " + tag,
             lambda y=y, n=n_x: hip.hipMemsetAsync(ctypes.c_void_p(y.data_ptr()), 0, 4 * n,
                                                    ctypes.c_void_p(stream.cuda_stream)), 4 * n_x),
            ("copy fp32 y -> y2 (read 1 : write 1), " + tag, lambda y=y, y2=y2: y2.copy_(y), 8 * n_x),
            ("convert bf16 x -> fp32 y (read 1 : write 2), " + tag, lambda y=y, xb=xb: y.copy_(xb), 6 * n_x),
        ]
    for name, fn, nbytes in ops:
        for _ in range(20):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3 / reps
        print(json.dumps({"op": name, "bytes": nbytes, "us": round(t * 1e6, 2),
                          "TB/s": round(nbytes / t / 1e12, 3), "frac_of_8TB/s": round(nbytes / t / 8e12, 3)}),
              flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this engine has no multi-GPU path "
              "(--gpus %d requested)." % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    if args.stream_probe:
        stream_probe()
        return
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n, "dispatches": 3}))
        return
    from cnn_convolution_forward_amd import synth

    wl = synth.ALL_WORKLOADS[args.workload]
    if args.backward and wl.dtype != "bf16":
        print("the backward pass takes bf16 inputs; %s is %s" % (wl.name, wl.dtype), file=sys.stderr)
        sys.exit(2)
    print("bench: %s route=%s steps=%d warmup=%d%s" % (wl.name, args.route, args.steps, args.warmup,
                                                       " backward" if args.backward else ""),
          file=sys.stderr, flush=True)
    options = (args.layout, args.out, args.relu)
    if args.backward and options != ("nchw", "f32", False):
        print("--layout/--out/--relu apply to the forward pass only", file=sys.stderr)
        sys.exit(2)
    if args.route == "explicit" and options != ("nchw", "f32", False):
        print("the explicit route takes NCHW, fp32 output, no ReLU", file=sys.stderr)
        sys.exit(2)
    runner, wall, gpu, main_t = measure(wl, args.route, args.steps, args.warmup, backward=args.backward,
                                        options=options, settle_ms=args.settle_ms)
    # backward: the data and the weight gradient each cost the forward's FLOP
    flops = wl.flops() * (2 if args.backward else 1)
    value = flops * args.steps / wall / 1e12
    dominant = "conv_bwd_weight_bf16" if args.backward else "convolution"
    kern_t = main_t
    if args.backward:
        bwd_us = {"conv_bwd_data_bf16": round(runner.pre_per[0] * 1e6, 3),
                  "conv_bwd_weight_bf16": round(main_t[0] * 1e6, 3)}
        if runner.pre_per[0] > main_t[0]:
            kern_t, dominant = runner.pre_per, "conv_bwd_data_bf16"
    out_bytes = 2 if args.out == "bf16" else 4
    counters, counters_src = counters_from_profiles(wl.name + ("_backward" if args.backward else ""), args.route)
    roof = roofline_entry(wl, args.route, kern_t[0], out_bytes, counters)
    roof.update({"traffic_source": counters_src, "kernel": dominant,
                 "kernel_avg_us": round(kern_t[0] * 1e6, 3),
                 "kernel_median_us": round(kern_t[1] * 1e6, 3),
                 "timing": ("the measured launch alone (%s), %d calls back to back in 5 batches, each batch "
                            "bracketed by one pair of HIP events on the library's stream; avg = total GPU time / "
                            "calls, median = median batch mean" % (
                                "conv2d_fwd_bf16_prepacked: the step's weight repack excluded"
                                if runner._pre is not None and not args.backward else dominant, args.steps))})
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "clock_settle": {"steps": runner.settle[0], "gpu_ms": round(runner.settle[1], 2),
                         "note": "untimed whole steps run before the warm-up steps until the GPU had been busy "
                                 "for --settle-ms (an idle GPU starts at a low clock)"},
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "gpu_ms_per_step": round(gpu / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded PCG64; x %s, w %s, b U[-1,1]%s)" % (
            "N(0,1)" if wl.x_dist == "normal" else "U[-1,1]",
            "U[-1,1]" if wl.dtype == "f32" else "N(0,1/sqrt(fan_in))",
            "; bf16 by RNE" if wl.dtype == "bf16" else ""),
        "config": describe(wl) | {"route": args.route, "pass": "backward" if args.backward else "forward",
                                  "layout": args.layout, "out_dtype": args.out, "relu": args.relu},
        "pct_bf16_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roof,
    }
    if runner._pre is not None and not args.backward:
        out["repack_us"] = round(runner.pre_per[0] * 1e6, 3)
    if args.route == "explicit" and runner._im2col is not None:
        im_t = _batched(runner.im2col, args.steps)
        im_bytes = int(np.prod(wl.x_shape)) * 2 + xcol_bytes(wl)
        out["im2col"] = {"bound": "hbm", "achieved": round(im_bytes / im_t[0] / 1e9, 2), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(im_bytes / im_t[0] / 1e9 / PEAK_HBM_GBS, 4),
                         "kernel_avg_us": round(im_t[0] * 1e6, 3), "algorithmic_bytes": im_bytes,
                         "xcol_over_x": round(xcol_bytes(wl) / (int(np.prod(wl.x_shape)) * 2), 3),
                         "note": "the explicit route's im2col kernel alone: x read once, X_col written once"}
    if not args.no_cold:
        n_cold = min(args.steps, 50)
        c_step, c_main = time_cold(runner, n_cold)
        out["cold_cache"] = {
            "steps": n_cold, "flush_bytes_between_steps": 512 << 20,
            "step_median_us": round(float(np.median(c_step)) * 1e6, 3),
            "step_min_us": round(float(np.min(c_step)) * 1e6, 3),
            "kernel_median_us": round(float(np.median(c_main)) * 1e6, 3),
            "kernel_min_us": round(float(np.min(c_main)) * 1e6, 3),
            "value": round(flops / float(np.median(c_step)) / 1e12, 3),
            "note": "the same steps, each after a 512 MiB scratch buffer is read outside the events "
                    "(L2s and the memory-side cache evicted, clean); value from the median step"}
    if args.backward:
        out["roofline"]["timing"] += ("; per call (us): %s; the longer call is the roofline's kernel (db is inside "
                                      "conv_bwd_weight_bf16)" % json.dumps(bwd_us))
    if not args.no_cpu_baseline:
        if args.backward:
            out["cpu_baseline"] = cpu_baseline_backward(wl, runner, args.cpu_sample_images or 2)
        else:
            n = args.cpu_sample_images or wl.N
            out["cpu_baseline"] = cpu_baseline(wl, runner, n)
    print(json.dumps(out), flush=True)
    if args.report:
        report_all(max(5, args.steps // 5), max(2, args.warmup // 2))


if __name__ == "__main__":
    main()
