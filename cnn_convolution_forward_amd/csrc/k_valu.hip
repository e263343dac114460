// k_valu.hip -- direct convolution on the vector ALUs (fp32 FMA; bf16 pairs
// through v_dot2_f32_bf16 in the LDS-staged bf16 kernel).
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
// reduction is too short for the matrix cores.  For bf16 inputs in NCHW with
// groups 1 the LDS-staged kernel takes two reduction indices per instruction
// (v_dot2_f32_bf16: both bf16 products, exact in fp32, added to the fp32
// accumulator); the fp32 path stays on fp32 FMA.
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

// LDS-staged variant (NCHW, groups 1, the block's fp32 weights plus a tap
// table within 64 KB of LDS): a workgroup of 256 threads takes 256 * PX
// consecutive output pixels (PX a thread, 256 apart) and OCB output
// channels.  The block's weights go to LDS once, as fp32, tap-major
// ([C_in * K^dims][OCB], zeros past C_out), with a table of each reduction
// index's (input channel, kd, kh, kw) offsets.  A thread walks the reduction
// in chunks of kChunk taps: it first loads the chunk's input values for its
// PX pixels (all in flight at once; zero outside the input, through a buffer
// resource, so no branch per tap), then for each tap reads the OCB weights as
// broadcast 16-byte LDS reads (every lane of a wave reads the same address)
// and does PX * OCB FMAs.  Launched with PX = 1 and OCB = 64 (16 for
// layers of at most 16 channels): on the stem layer (C_in = 3, 3x3, stride 2,
// 64 channels) that took 52 us against 72-218 us for (OCB, PX) = (64, 2),
// (32, 2..4), (16, 4..8): the per-pixel address work and the lower occupancy
// of more pixels a thread cost more than the weight reads they share.  The
// general kernel took 147 us.
constexpr int kLdsWBytes = 64 * 1024;
constexpr int kChunk = 8;

template <typename T, int OCB, int PX>
__global__ __launch_bounds__(kThreads)
void direct_lds_kernel(Shape sh, const T *__restrict__ x, const T *__restrict__ w,
                       const float *__restrict__ bias, float *__restrict__ y, int64_t P) {
    extern __shared__ float4 wsm4[];
    float *const wsm = reinterpret_cast<float *>(wsm4);
    const int taps = (int)sh.taps();
    const int red = sh.C * taps;                         // reduction length
    int4 *const ktab = reinterpret_cast<int4 *>(wsm + (size_t)red * OCB);
    const int oc0 = blockIdx.y * OCB;
    // the weights, 8 loads a thread in flight before their LDS stores
    for (int i0 = 0; i0 < red * OCB; i0 += 8 * kThreads) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kThreads + threadIdx.x;
            const int k = i / OCB, o = i - k * OCB;
            v[u] = (i < red * OCB && oc0 + o < sh.Co) ? ld(w, (int64_t)(oc0 + o) * red + k) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kThreads + threadIdx.x;
            if (i < red * OCB) wsm[i] = v[u];
        }
    }
    for (int k = threadIdx.x; k < red; k += kThreads) {
        // k = ((ic*Kd + kd)*K + kh)*K + kw
        const int kw = k % sh.K, kh = (k / sh.K) % sh.K, kd = (k / (sh.K * sh.K)) % sh.Kd, ic = k / taps;
        ktab[k] = make_int4(ic, kd * sh.dild, kh * sh.dil, kw * sh.dil);
    }
    __syncthreads();
    const int64_t plane = sh.out_plane();
    const int64_t HW = (int64_t)sh.H * sh.W, DHW = HW * sh.D;
    // per pixel: its image's input resource and the window origin
    __amdgpu_buffer_rsrc_t xr[PX];
    int id0[PX], ih0[PX], iw0[PX];
    int64_t yb[PX];
    bool live[PX];
#pragma unroll
    for (int q = 0; q < PX; ++q) {
        const int64_t px = ((int64_t)blockIdx.x * PX + q) * kThreads + threadIdx.x;
        live[q] = px < P;
        int64_t t = live[q] ? px : 0;
        const int ow = (int)(t % sh.Wo); t /= sh.Wo;
        const int oh = (int)(t % sh.Ho); t /= sh.Ho;
        const int od = (int)(t % sh.Do); t /= sh.Do;
        const int64_t n = t;
        id0[q] = od * sh.sd - sh.pd; ih0[q] = oh * sh.s - sh.p; iw0[q] = ow * sh.s - sh.p;
        xr[q] = make_rsrc(x + n * sh.C * DHW, (uint32_t)(sh.C * DHW * sizeof(T)));
        yb[q] = n * sh.Co * plane + ((live[q] ? px : 0) - n * plane);
    }

    float acc[PX][OCB];
#pragma unroll
    for (int q = 0; q < PX; ++q)
#pragma unroll
        for (int o = 0; o < OCB; ++o) acc[q][o] = 0.f;
    for (int k0 = 0; k0 < red; k0 += kChunk) {
        float xv[kChunk][PX];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const int4 e = ktab[k0 + j < red ? k0 + j : red - 1];
#pragma unroll
            for (int q = 0; q < PX; ++q) {
                const int id = id0[q] + e.y, ih = ih0[q] + e.z, iw = iw0[q] + e.w;
                const bool in = live[q] && k0 + j < red && id >= 0 && id < sh.D && ih >= 0 && ih < sh.H && iw >= 0 &&
                                iw < sh.W;
                const uint32_t off =
                    in ? (uint32_t)((e.x * DHW + (int64_t)id * HW + (int64_t)ih * sh.W + iw) * sizeof(T)) : kOob;
                if constexpr (sizeof(T) == 2)
                    xv[j][q] = bf16_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(xr[q], (int)off, 0, 0));
                else
                    xv[j][q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr[q], (int)off, 0, 0));
            }
        }
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            if (k0 + j >= red) break;                    // uniform
            const float4 *wk = wsm4 + (k0 + j) * (OCB / 4);
#pragma unroll
            for (int o4 = 0; o4 < OCB / 4; ++o4) {
                const float4 wv = wk[o4];
#pragma unroll
                for (int q = 0; q < PX; ++q) {
                    acc[q][4 * o4 + 0] = __builtin_fmaf(xv[j][q], wv.x, acc[q][4 * o4 + 0]);
                    acc[q][4 * o4 + 1] = __builtin_fmaf(xv[j][q], wv.y, acc[q][4 * o4 + 1]);
                    acc[q][4 * o4 + 2] = __builtin_fmaf(xv[j][q], wv.z, acc[q][4 * o4 + 2]);
                    acc[q][4 * o4 + 3] = __builtin_fmaf(xv[j][q], wv.w, acc[q][4 * o4 + 3]);
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < PX; ++q) {
        if (!live[q]) continue;
#pragma unroll
        for (int o = 0; o < OCB; ++o) {
            const int oc = oc0 + o;
            if (oc < sh.Co)
                store_out(y, yb[q] + (int64_t)oc * plane, acc[q][o] + (bias ? bias[oc] : 0.f), sh.out_bf16, sh.relu);
        }
    }
}

// bf16 form of the LDS-staged kernel with two reduction indices per
// instruction: v_dot2_f32_bf16 multiplies a pair of bf16 inputs by a pair of
// bf16 weights and adds both products to an fp32 accumulator, so the 27-long
// reduction of the stem layer is 14 instructions per output instead of 27
// FMAs, and the weights stay bf16 in LDS ([pairs][OCB] dwords; a pair is W_row
// indices 2j, 2j + 1, the second zero past an odd reduction length), so a
// broadcast 16-byte read serves 4 channels x 2 taps.  The inputs of a pair are
// two 2-byte buffer loads (0 outside the input), packed into one dword.
// Stem layer: 43.5 us against 54.2 us for the fp32-FMA kernel on bf16 inputs,
// 3D layer 99.5 against 125.9 us.  Measured and not kept: 2 pixels a thread
// (67 us), 32 channels a block (43.6 / 116 us), 2 or 8 pairs of loads in flight
// (no change), and the outputs staged in LDS so a wave stores 1 KB of one
// plane (47.4 us; a build without any stores took 28.4 us).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int OCB, int PX, int kChunk2>
__global__ __launch_bounds__(kThreads)
void direct_dot2_kernel(Shape sh, const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                        const float *__restrict__ bias, float *__restrict__ y, int64_t P) {
    extern __shared__ uint4 wsm_u4[];
    uint32_t *const wsm = reinterpret_cast<uint32_t *>(wsm_u4);
    const int taps = (int)sh.taps();
    const int red = sh.C * taps;                         // reduction length
    const int red2 = (red + 1) / 2;                      // pairs
    int4 *const ktab = reinterpret_cast<int4 *>(wsm + (size_t)red2 * OCB);
    const int oc0 = blockIdx.y * OCB;
    for (int i = threadIdx.x; i < red2 * OCB; i += kThreads) {
        const int j = i / OCB, o = i - j * OCB;
        uint32_t v = 0;
        if (oc0 + o < sh.Co) {
            const uint16_t *wr = w + (int64_t)(oc0 + o) * red;
            v = wr[2 * j];
            if (2 * j + 1 < red) v |= (uint32_t)wr[2 * j + 1] << 16;
        }
        wsm[i] = v;
    }
    for (int k = threadIdx.x; k < 2 * red2; k += kThreads) {
        // k = ((ic*Kd + kd)*K + kh)*K + kw; the pad index past an odd length
        // gets an input channel past the end (its loads read 0)
        const int kw = k % sh.K, kh = (k / sh.K) % sh.K, kd = (k / (sh.K * sh.K)) % sh.Kd, ic = k / taps;
        ktab[k] = make_int4(k < red ? ic : -1, kd * sh.dild, kh * sh.dil, kw * sh.dil);
    }
    __syncthreads();
    const int64_t plane = sh.out_plane();
    const int64_t HW = (int64_t)sh.H * sh.W, DHW = HW * sh.D;
    __amdgpu_buffer_rsrc_t xr[PX];
    int id0[PX], ih0[PX], iw0[PX];
    int64_t yb[PX];
    bool live[PX];
#pragma unroll
    for (int q = 0; q < PX; ++q) {
        const int64_t px = ((int64_t)blockIdx.x * PX + q) * kThreads + threadIdx.x;
        live[q] = px < P;
        int64_t t = live[q] ? px : 0;
        const int ow = (int)(t % sh.Wo); t /= sh.Wo;
        const int oh = (int)(t % sh.Ho); t /= sh.Ho;
        const int od = (int)(t % sh.Do); t /= sh.Do;
        const int64_t n = t;
        id0[q] = od * sh.sd - sh.pd; ih0[q] = oh * sh.s - sh.p; iw0[q] = ow * sh.s - sh.p;
        xr[q] = make_rsrc(x + n * sh.C * DHW, (uint32_t)(sh.C * DHW * 2));
        yb[q] = n * sh.Co * plane + ((live[q] ? px : 0) - n * plane);
    }

    float acc[PX][OCB];
#pragma unroll
    for (int q = 0; q < PX; ++q)
#pragma unroll
        for (int o = 0; o < OCB; ++o) acc[q][o] = 0.f;
    auto xoff = [&](const int4 &e, int q) -> uint32_t {
        const int id = id0[q] + e.y, ih = ih0[q] + e.z, iw = iw0[q] + e.w;
        const bool in = live[q] && e.x >= 0 && id >= 0 && id < sh.D && ih >= 0 && ih < sh.H && iw >= 0 && iw < sh.W;
        return in ? (uint32_t)((e.x * DHW + (int64_t)id * HW + (int64_t)ih * sh.W + iw) * 2) : kOob;
    };
    for (int j0 = 0; j0 < red2; j0 += kChunk2) {
        uint32_t xp[kChunk2][PX];
#pragma unroll
        for (int j = 0; j < kChunk2; ++j) {
            const int jj = j0 + j < red2 ? j0 + j : red2 - 1;
            const int4 e0 = ktab[2 * jj], e1 = ktab[2 * jj + 1];
#pragma unroll
            for (int q = 0; q < PX; ++q) {
                const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(xr[q], (int)xoff(e0, q), 0, 0);
                const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(xr[q], (int)xoff(e1, q), 0, 0);
                xp[j][q] = (lo & 0xffffu) | (hi << 16);
            }
        }
#pragma unroll
        for (int j = 0; j < kChunk2; ++j) {
            if (j0 + j >= red2) break;                   // uniform
            const uint4 *wk = wsm_u4 + (j0 + j) * (OCB / 4);
#pragma unroll
            for (int o4 = 0; o4 < OCB / 4; ++o4) {
                const uint4 wv = wk[o4];
#pragma unroll
                for (int q = 0; q < PX; ++q) {
                    const bf16x2_t a = __builtin_bit_cast(bf16x2_t, xp[j][q]);
                    acc[q][4 * o4 + 0] = __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, wv.x), acc[q][4 * o4 + 0], false);
                    acc[q][4 * o4 + 1] = __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, wv.y), acc[q][4 * o4 + 1], false);
                    acc[q][4 * o4 + 2] = __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, wv.z), acc[q][4 * o4 + 2], false);
                    acc[q][4 * o4 + 3] = __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, wv.w), acc[q][4 * o4 + 3], false);
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < PX; ++q) {
        if (!live[q]) continue;
#pragma unroll
        for (int o = 0; o < OCB; ++o) {
            const int oc = oc0 + o;
            if (oc < sh.Co)
                store_out(y, yb[q] + (int64_t)oc * plane, acc[q][o] + (bias ? bias[oc] : 0.f), sh.out_bf16, sh.relu);
        }
    }
}

template <int OCB, int PX, int CH = 4>
hipError_t launch_direct_dot2(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias, float *y,
                              hipStream_t st) {
    const int64_t P = sh.pixels();
    const int nblk = (sh.Co + OCB - 1) / OCB;
    const int64_t red2 = ((int64_t)sh.C * sh.taps() + 1) / 2;
    const size_t lds = (size_t)red2 * (OCB * 4 + 32);
    dim3 grid((unsigned)((P + (int64_t)kThreads * PX - 1) / ((int64_t)kThreads * PX)), (unsigned)nblk);
    hipLaunchKernelGGL((direct_dot2_kernel<OCB, PX, CH>), grid, dim3(kThreads), lds, st, sh, x, w, bias, y, P);
    return hipGetLastError();
}

template <typename T, int OCB, int PX>
hipError_t launch_direct_lds(const Shape &sh, const T *x, const T *w, const float *bias, float *y, hipStream_t st) {
    const int64_t P = sh.pixels();
    const int nblk = (sh.Co + OCB - 1) / OCB;
    const size_t lds = (size_t)sh.C * sh.taps() * (OCB * 4 + 16);
    dim3 grid((unsigned)((P + (int64_t)kThreads * PX - 1) / ((int64_t)kThreads * PX)), (unsigned)nblk);
    hipLaunchKernelGGL((direct_lds_kernel<T, OCB, PX>), grid, dim3(kThreads), lds, st, sh, x, w, bias, y, P);
    return hipGetLastError();
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
// The LDS-staged kernel where it applies (NCHW, groups 1, the block's fp32
// weights within 64 KB of LDS, grid.y within its limit): 64 channels a block,
// or 16 for layers of at most 16 output channels; else the general kernel,
// with a channel block of 8, or the smallest power of two that holds a
// smaller group.
template <typename T>
hipError_t launch_direct(const Shape &sh, const T *x, const T *w, const float *bias, float *y,
                         hipStream_t st) {
    // (one image's input within a buffer resource's 2^31-byte offset range)
    if (!sh.nhwc && sh.G == 1 && (int64_t)sh.C * sh.in_plane() * (int64_t)sizeof(T) < (INT64_C(1) << 31)) {
        const int64_t red = (int64_t)sh.C * sh.taps();
        if constexpr (sizeof(T) == 2) {
            const int64_t red2 = (red + 1) / 2;
            if (sh.Co <= 16 && red2 * (16 * 4 + 32) <= kLdsWBytes) return launch_direct_dot2<16, 1>(sh, x, w, bias, y, st);
            if (sh.Co > 16 && red2 * (64 * 4 + 32) <= kLdsWBytes && (sh.Co + 63) / 64 <= 65535)
                return launch_direct_dot2<64, 1>(sh, x, w, bias, y, st);
        }
        if (sh.Co <= 16 && red * (16 * 4 + 16) <= kLdsWBytes) return launch_direct_lds<T, 16, 1>(sh, x, w, bias, y, st);
        if (sh.Co > 16 && red * (64 * 4 + 16) <= kLdsWBytes && (sh.Co + 63) / 64 <= 65535)
            return launch_direct_lds<T, 64, 1>(sh, x, w, bias, y, st);
    }
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
