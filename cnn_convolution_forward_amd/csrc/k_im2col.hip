// k_im2col.hip -- explicit im2col: materialise X_col in device memory.
//
// X_col has C_in*K^dims rows and N*Do*Ho*Wo columns, row-major, bf16.  Row
// r = ((ic*Kd + kd)*K + kh)*K + kw; column j = ((n*Do + od)*Ho + oh)*Wo + ow;
// the entry is x at (od*sd+kd*dd-pd, oh*s+kh*d-p, ow*s+kw*d-p), or 0 when that
// coordinate is outside the input ("Why use matrix multiplication for
// convolution", 2.2 and 3.1; zero padding by bounds checks, "Hand-writing
// Conv2D", 1.2; taps d apart under dilation, "PyTorch tensor products and
// conv2d/conv3d dimension semantics", 4.2).  Groups do not change X_col: group
// g multiplies its own block of C_in/G * K^dims consecutive rows.  It is a
// pure copy, so the result is exact.
//
// Mapping: a thread owns one row r and 8 consecutive columns, so a wave writes
// 64 x 16 B = 1 KB contiguous along j (the pixel axis) and, for stride 1, reads
// consecutive input columns.  X_col is K^dims times larger than x: this kernel
// exists to measure that blow-up.
#include "conv_internal.h"

namespace convfwd {
namespace {

constexpr int kThreads = 256;
constexpr int kColsPerThread = 8;

__global__ __launch_bounds__(kThreads)
void im2col_bf16_kernel(Shape sh, const uint16_t *__restrict__ x, uint16_t *__restrict__ xcol,
                        int64_t J, int rows) {
    const int64_t j0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kColsPerThread;
    if (j0 >= J) return;
    const int K = sh.K, Kd = sh.Kd, Wo = sh.Wo, Ho = sh.Ho, Do = sh.Do;
    // Column j0 -> (n, od, oh, ow); advanced with carries below.
    int64_t t = j0;
    int ow0 = (int)(t % Wo); t /= Wo;
    int oh0 = (int)(t % Ho); t /= Ho;
    int od0 = (int)(t % Do); t /= Do;
    int n0 = (int)t;
    const bool vec = (J % kColsPerThread) == 0;      // rows 16-byte aligned, full 8-column groups
    for (int r = blockIdx.y; r < rows; r += gridDim.y) {
        int kw = r % K, q = r / K;
        int kh = q % K; q /= K;
        int kd = q % Kd;
        int ic = q / Kd;
        int ow = ow0, oh = oh0, od = od0, n = n0;
        uint16_t v[kColsPerThread];
#pragma unroll
        for (int e = 0; e < kColsPerThread; ++e) {
            uint16_t val = 0;
            if (n < sh.N) {
                int id = od * sh.sd + kd * sh.dild - sh.pd;
                int ih = oh * sh.s + kh * sh.dil - sh.p;
                int iw = ow * sh.s + kw * sh.dil - sh.p;
                if (0 <= id && id < sh.D && 0 <= ih && ih < sh.H && 0 <= iw && iw < sh.W)
                    val = x[(((int64_t)n * sh.C + ic) * sh.D + id) * ((int64_t)sh.H * sh.W) +
                            (int64_t)ih * sh.W + iw];
            }
            v[e] = val;
            if (++ow == Wo) { ow = 0; if (++oh == Ho) { oh = 0; if (++od == Do) { od = 0; ++n; } } }
        }
        uint16_t *dst = xcol + (int64_t)r * J + j0;
        if (vec) {
            uint4 pk;
            pk.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
            pk.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
            pk.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
            pk.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
            *reinterpret_cast<uint4 *>(dst) = pk;
        } else {
#pragma unroll
            for (int e = 0; e < kColsPerThread; ++e)
                if (j0 + e < J) dst[e] = v[e];
        }
    }
}

// The five dwords that start q dwords into d[0..15] (q uniform across the
// wave: one scalar branch, constant register indices in each arm).
__device__ __forceinline__ void pick5(const uint32_t (&d)[16], int q, uint32_t (&o)[5]) {
    switch (q) {
#define IM2COL_PICK(Q) case Q: o[0] = d[Q]; o[1] = d[Q + 1]; o[2] = d[Q + 2]; o[3] = d[Q + 3]; o[4] = d[Q + 4]; break;
        IM2COL_PICK(0) IM2COL_PICK(1) IM2COL_PICK(2) IM2COL_PICK(3) IM2COL_PICK(4) IM2COL_PICK(5)
        IM2COL_PICK(6) IM2COL_PICK(7) IM2COL_PICK(8) IM2COL_PICK(9) IM2COL_PICK(10)
        default: IM2COL_PICK(11)
#undef IM2COL_PICK
    }
}

// 2D, stride 1, W % 8 == 0, Wo % 8 == 0, (K - 1) * d <= 16, 16-byte aligned x
// and X_col.  Row r = (ic, kh, kw) of X_col, over image n's columns, is input
// plane (n, ic) shifted by (kh*d - p, kw*d - p), zeros outside it.  A thread
// takes 8 consecutive columns (one output row oh, columns ow0 .. ow0 + 7;
// they never straddle rows since Wo % 8 == 0) of all K*K rows of one input
// channel: for each kh it loads input row ih = oh + kh*d - p as the four
// aligned 16-byte chunks from a0 = floor((ow0 - p) / 8) * 8 on (32 elements,
// enough for the 8 + (K-1)*d needed; a chunk lies wholly inside the row or
// wholly outside since W % 8 == 0, and one outside, or a row outside the
// image, reads as zeros), then writes the K rows kw as 16-byte stores of
// the elements shifted by t = kw*d + (ow0 - p - a0) -- the same t for the
// whole wave, since ow0 is a multiple of 8.  K*K stores and 4K loads a
// thread (the loads mostly hit L2: the K*K rows of a channel reuse them).
__global__ __launch_bounds__(kThreads)
void im2col_s1_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ xcol, int C, int H, int W, int Ho,
                      int Wo, int K, int p, int d, int64_t J) {
    const int64_t j0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kColsPerThread;
    if (j0 >= J) return;
    const int ic = blockIdx.y;
    const int64_t plane = (int64_t)Ho * Wo;
    const int n = (int)(j0 / plane);
    const int q0 = (int)(j0 - n * plane);
    const int oh = q0 / Wo, ow0 = q0 - oh * Wo;
    const int a0 = ((ow0 - p) >> 3) << 3;                 // floor to a multiple of 8 (arithmetic shift)
    const int s0 = ow0 - p - a0;                          // 0 .. 7, uniform
    const uint16_t *plane_x = x + (int64_t)(n * C + ic) * H * W;
    uint16_t *dst = xcol + (int64_t)ic * K * K * J + j0;
    for (int kh = 0; kh < K; ++kh) {
        const int ih = oh + kh * d - p;
        uint32_t dw[16];
        const bool row_in = ih >= 0 && ih < H;
        const uint16_t *row = plane_x + (int64_t)(row_in ? ih : 0) * W;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int a = a0 + 8 * c;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row_in && a >= 0 && a < W) v = *reinterpret_cast<const uint4 *>(row + a);
            dw[4 * c + 0] = v.x; dw[4 * c + 1] = v.y; dw[4 * c + 2] = v.z; dw[4 * c + 3] = v.w;
        }
        for (int kw = 0; kw < K; ++kw) {
            const int t = kw * d + s0;                    // element shift, <= 16 + 7
            uint32_t o[5];
            pick5(dw, t >> 1, o);
            const int sh = (t & 1) * 2;                   // bytes
            const uint4 out = make_uint4(__builtin_amdgcn_alignbyte(o[1], o[0], sh),
                                         __builtin_amdgcn_alignbyte(o[2], o[1], sh),
                                         __builtin_amdgcn_alignbyte(o[3], o[2], sh),
                                         __builtin_amdgcn_alignbyte(o[4], o[3], sh));
            *reinterpret_cast<uint4 *>(dst + (int64_t)(kh * K + kw) * J) = out;
        }
    }
}

}  // namespace

hipError_t launch_im2col_bf16(const Shape &sh, const uint16_t *x, uint16_t *xcol, hipStream_t st) {
    const int64_t J = sh.pixels();
    const int rows = (int)sh.xcol_rows();
    if (sh.ndim == 2 && sh.s == 1 && sh.W % 8 == 0 && sh.Wo % 8 == 0 && (sh.K - 1) * sh.dil <= 16 && !sh.nhwc &&
        ((uintptr_t)x % 16) == 0 && ((uintptr_t)xcol % 16) == 0 && sh.C <= 65535) {
        const int64_t groups = J / kColsPerThread;
        dim3 grid((unsigned)((groups + kThreads - 1) / kThreads), (unsigned)sh.C);
        hipLaunchKernelGGL(im2col_s1_kernel, grid, dim3(kThreads), 0, st, x, xcol, sh.C, sh.H, sh.W, sh.Ho, sh.Wo,
                           sh.K, sh.p, sh.dil, J);
        return hipGetLastError();
    }
    const int64_t groups = (J + kColsPerThread - 1) / kColsPerThread;
    dim3 grid((unsigned)((groups + kThreads - 1) / kThreads), (unsigned)(rows < 65535 ? rows : 65535));
    hipLaunchKernelGGL(im2col_bf16_kernel, grid, dim3(kThreads), 0, st, sh, x, xcol, J, rows);
    return hipGetLastError();
}

}  // namespace convfwd
