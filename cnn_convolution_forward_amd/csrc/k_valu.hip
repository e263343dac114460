// k_valu.hip -- direct convolution on the vector ALUs (fp32 FMA).
//
// The direct form loops over output positions and, for each, over the (ic, kd,
// kh, kw) taps with bounds checks ("Hand-writing Conv2D", 2.1; "Why use matrix
// multiplication for convolution", 5.2: no extra memory).  Each output is
// independent, so a thread owns one output pixel and OCB output channels.  The
// OCB weights of a tap are the same for the whole workgroup (blockIdx.y picks
// the channel group), so they are fetched with scalar loads and broadcast;
// x is read once per tap and reused across the OCB channels.
//
// With groups G, output channel oc reads the C_in/G input channels of group
// oc / (C_out/G); blockIdx.y enumerates (group, channel block) pairs so that
// the OCB channels of a block share one group and one input read per tap.
// Dilation d places the taps d inputs apart ("PyTorch tensor products and
// conv2d/conv3d dimension semantics", 4.2-4.3).
//
// x and y may be channels-last (sh.nhwc), and the store may apply ReLU and
// round to bf16 (sh.relu, sh.out_bf16).
//
// Used for the fp32 path and for thin layers (C_in*K^dims small) where the
// reduction is too short for the matrix cores.
#include "conv_internal.h"
#include "mfma_common.h"

namespace convfwd {
namespace {

constexpr int kThreads = 256;

template <typename T> __device__ __forceinline__ float ld(const T *p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
}

template <typename T, int OCB>
__global__ __launch_bounds__(kThreads)
void direct_kernel(Shape sh, const T *__restrict__ x, const T *__restrict__ w,
                   const float *__restrict__ bias, float *__restrict__ y, int64_t P, int nblk) {
    const int64_t px = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (px >= P) return;
    const int Cog = sh.Co / sh.G, Cg = sh.C / sh.G;
    const int64_t plane = sh.out_plane();
    int64_t t = px;
    const int ow = (int)(t % sh.Wo); t /= sh.Wo;
    const int oh = (int)(t % sh.Ho); t /= sh.Ho;
    const int od = (int)(t % sh.Do); t /= sh.Do;
    const int64_t n = t;
    const int64_t HW = (int64_t)sh.H * sh.W;
    const int64_t taps = sh.taps();
    const int id0 = od * sh.sd - sh.pd, ih0 = oh * sh.s - sh.p, iw0 = ow * sh.s - sh.p;
    const int64_t q = px - n * plane;
    // NCHW: channel planes; NHWC: channel fastest (x and y)
    const int64_t cstride = sh.nhwc ? 1 : sh.in_plane(), pstride = sh.nhwc ? sh.C : 1;
    const int64_t ocs = sh.nhwc ? 1 : plane;
    const int64_t yb = n * sh.Co * plane + (sh.nhwc ? q * sh.Co : q);

    // (group, channel block) pairs, nblk blocks per group, strided over grid.y
    for (int by = blockIdx.y; by < sh.G * nblk; by += gridDim.y) {
        const int grp = by / nblk;
        const int ocl0 = (by - grp * nblk) * OCB;      // first channel of the block inside its group
        const int oc0 = grp * Cog + ocl0;
        const T *xn = x + n * sh.C * sh.in_plane() + (int64_t)grp * Cg * cstride;

        float acc[OCB];
#pragma unroll
        for (int o = 0; o < OCB; ++o) acc[o] = 0.f;

        for (int ic = 0; ic < Cg; ++ic) {
            const T *xc = xn + (int64_t)ic * cstride;
            const T *wc = w + (int64_t)ic * taps;
            for (int kd = 0; kd < sh.Kd; ++kd) {
                const int id = id0 + kd * sh.dild;
                if (id < 0 || id >= sh.D) continue;
                for (int kh = 0; kh < sh.K; ++kh) {
                    const int ih = ih0 + kh * sh.dil;
                    if (ih < 0 || ih >= sh.H) continue;
                    for (int kw = 0; kw < sh.K; ++kw) {
                        const int iw = iw0 + kw * sh.dil;
                        if (iw < 0 || iw >= sh.W) continue;
                        const float xv = ld(xc, ((int64_t)id * HW + (int64_t)ih * sh.W + iw) * pstride);
                        const int64_t tap = ((int64_t)kd * sh.K + kh) * sh.K + kw;
#pragma unroll
                        for (int o = 0; o < OCB; ++o) {
                            // clamp to the group's last channel: reads stay in bounds
                            const int oc = ocl0 + o < Cog ? oc0 + o : grp * Cog + Cog - 1;
                            acc[o] = __builtin_fmaf(xv, ld(wc, (int64_t)oc * Cg * taps + tap), acc[o]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int o = 0; o < OCB; ++o) {
            const int oc = oc0 + o;
            if (ocl0 + o < Cog) store_out(y, yb + (int64_t)oc * ocs, acc[o] + (bias ? bias[oc] : 0.f), sh.out_bf16, sh.relu);
        }
    }
}

template <typename T, int OCB>
hipError_t launch_direct_ocb(const Shape &sh, const T *x, const T *w, const float *bias, float *y,
                             hipStream_t st) {
    const int64_t P = sh.pixels();
    const int nblk = (sh.Cog() + OCB - 1) / OCB;
    const int64_t gy = (int64_t)sh.G * nblk;                   // < 2^31: nblk <= Cog and G * Cog = Co
    dim3 grid((unsigned)((P + kThreads - 1) / kThreads), (unsigned)(gy < 65535 ? gy : 65535));
    hipLaunchKernelGGL((direct_kernel<T, OCB>), grid, dim3(kThreads), 0, st, sh, x, w, bias, y, P, nblk);
    return hipGetLastError();
}

// Channel block: 8, or the smallest power of two that holds a smaller group.
template <typename T>
hipError_t launch_direct(const Shape &sh, const T *x, const T *w, const float *bias, float *y,
                         hipStream_t st) {
    const int cog = sh.Cog();
    if (cog >= 5) return launch_direct_ocb<T, 8>(sh, x, w, bias, y, st);
    if (cog >= 3) return launch_direct_ocb<T, 4>(sh, x, w, bias, y, st);
    if (cog == 2) return launch_direct_ocb<T, 2>(sh, x, w, bias, y, st);
    return launch_direct_ocb<T, 1>(sh, x, w, bias, y, st);
}

}  // namespace

hipError_t launch_valu_f32(const Shape &sh, const float *x, const float *w, const float *bias,
                           float *y, hipStream_t st) {
    return launch_direct<float>(sh, x, w, bias, y, st);
}

hipError_t launch_valu_generic_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w,
                                    const float *bias, float *y, hipStream_t st) {
    return launch_direct<uint16_t>(sh, x, w, bias, y, st);
}

}  // namespace convfwd
