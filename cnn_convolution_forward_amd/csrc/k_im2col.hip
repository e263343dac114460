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

}  // namespace

hipError_t launch_im2col_bf16(const Shape &sh, const uint16_t *x, uint16_t *xcol, hipStream_t st) {
    const int64_t J = sh.pixels();
    const int rows = (int)sh.xcol_rows();
    const int64_t groups = (J + kColsPerThread - 1) / kColsPerThread;
    dim3 grid((unsigned)((groups + kThreads - 1) / kThreads), (unsigned)(rows < 65535 ? rows : 65535));
    hipLaunchKernelGGL(im2col_bf16_kernel, grid, dim3(kThreads), 0, st, sh, x, xcol, J, rows);
    return hipGetLastError();
}

}  // namespace convfwd
