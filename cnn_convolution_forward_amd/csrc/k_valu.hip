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
                   const float *__restrict__ bias, float *__restrict__ y, int64_t P) {
    const int64_t px = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int oc0 = blockIdx.y * OCB;
    if (px >= P) return;
    const int64_t plane = sh.out_plane();
    int64_t t = px;
    const int ow = (int)(t % sh.Wo); t /= sh.Wo;
    const int oh = (int)(t % sh.Ho); t /= sh.Ho;
    const int od = (int)(t % sh.Do); t /= sh.Do;
    const int64_t n = t;
    const int64_t HW = (int64_t)sh.H * sh.W;
    const int64_t taps = sh.taps();
    const T *xn = x + n * sh.C * sh.in_plane();

    float acc[OCB];
#pragma unroll
    for (int o = 0; o < OCB; ++o) acc[o] = 0.f;

    const int id0 = od * sh.sd - sh.pd, ih0 = oh * sh.s - sh.p, iw0 = ow * sh.s - sh.p;
    for (int ic = 0; ic < sh.C; ++ic) {
        const T *xc = xn + (int64_t)ic * sh.in_plane();
        const T *wc = w + (int64_t)ic * taps;
        for (int kd = 0; kd < sh.Kd; ++kd) {
            const int id = id0 + kd;
            if (id < 0 || id >= sh.D) continue;
            for (int kh = 0; kh < sh.K; ++kh) {
                const int ih = ih0 + kh;
                if (ih < 0 || ih >= sh.H) continue;
                for (int kw = 0; kw < sh.K; ++kw) {
                    const int iw = iw0 + kw;
                    if (iw < 0 || iw >= sh.W) continue;
                    const float xv = ld(xc, (int64_t)id * HW + (int64_t)ih * sh.W + iw);
                    const int64_t tap = ((int64_t)kd * sh.K + kh) * sh.K + kw;
#pragma unroll
                    for (int o = 0; o < OCB; ++o) {
                        const int oc = oc0 + o < sh.Co ? oc0 + o : sh.Co - 1;   // clamp: reads stay in bounds
                        acc[o] = __builtin_fmaf(xv, ld(wc, (int64_t)oc * sh.C * taps + tap), acc[o]);
                    }
                }
            }
        }
    }
    float *yp = y + n * sh.Co * plane + (px - n * plane);
#pragma unroll
    for (int o = 0; o < OCB; ++o) {
        const int oc = oc0 + o;
        if (oc < sh.Co) yp[(int64_t)oc * plane] = acc[o] + (bias ? bias[oc] : 0.f);
    }
}

template <typename T>
hipError_t launch_direct(const Shape &sh, const T *x, const T *w, const float *bias, float *y,
                         hipStream_t st) {
    constexpr int OCB = 8;
    const int64_t P = sh.pixels();
    dim3 grid((unsigned)((P + kThreads - 1) / kThreads), (unsigned)((sh.Co + OCB - 1) / OCB));
    hipLaunchKernelGGL((direct_kernel<T, OCB>), grid, dim3(kThreads), 0, st, sh, x, w, bias, y, P);
    return hipGetLastError();
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
