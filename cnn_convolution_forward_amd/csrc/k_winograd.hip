// k_winograd.hip -- 3x3, stride-1 convolution by Winograd F(2x2, 3x3)
// ("Why use matrix multiplication for convolution", 5.1: (m+r-1)^2 = 16
// multiplications per 2x2 output block instead of m^2 r^2 = 36; 3x3 kernels,
// stride 1, dilation 1 only).  The transform matrices are the published
// minimal-filtering ones of F(2,3), nested for two dimensions:
//     B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1]
//     G   = [1 0 0; 1/2 1/2 1/2; 1/2 -1/2 1/2; 0 0 1]
//     A^T = [1 1 1 0; 0 1 -1 -1]
//
// Three kernels:
//  1. U[xi][k][c] = (G g[k][c] G^T)[xi], fp16, once per call;
//  2. V[xi][c/32][t][c%32] = (B^T d[c][t] B)[xi], fp16, for every 2x2 output
//     block t (channels in tiles of 32, so a tile's blocks are contiguous)
//     (its 4x4 input block d, zero outside the image) -- from LDS tiles of
//     32 channels x 32 blocks when C_in % 32 == 0 and W % 8 == 0, else one
//     thread per (block, 8 channels) straight from global memory;
//  3. for each of the 16 transform points xi the GEMM M[xi] = U[xi] @ V[xi]^T
//     (C_out x blocks, reduction over C_in) on v_mfma_f32_32x32x16_f16 with
//     fp32 accumulation, then, in the same workgroup, Y = A^T M A per block,
//     + bias, stored into y (NCHW, fp32 or bf16, optional ReLU), the last
//     block row/column cropped.
// fp16 rather than bf16 for U and V: the transformed operands are rounded
// before the products, and fp16's 11-bit significand keeps that error near
// 2^-11 of the transform-domain magnitudes (bf16's 8 bits would be 8x worse,
// the low-precision risk the page warns about).  fp16 spans only 2^-24 ..
// 65504 where bf16 spans fp32's range, so x and w are first scaled by powers
// of two: a pass over both finds max|x| and max|w|, and the transforms
// multiply by 2^kx and 2^kw chosen so that the transformed values stay below
// 2^13 (|V| <= 4 max|x|, |U| <= 2.25 max|w|), and the output transform
// multiplies by 2^-(kx + kw).  Scaling by a power of two is exact, so results
// within fp16's normal range are those of the unscaled transforms; only
// values more than ~2^27 below their tensor's largest magnitude become fp16
// subnormals.
//
// A GEMM workgroup computes 32 output channels x 32 blocks for all 16
// points: wave w owns points 4w..4w+3 (4 accumulator tiles), loads its
// operands straight from U and V in 16-byte pieces (8 consecutive input
// channels per lane, the MFMA layout), one stage of 16 channels ahead; the
// 16 x 32 x 32 results meet in LDS for the output transform.
#include "conv_internal.h"
#include "mfma_common.h"

namespace convfwd {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16_t mfma32x32x16_f16(const uint4 &a, const uint4 &b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ uint16_t f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// 0. The scale exponents.  mag[0], mag[1] receive the bit patterns of max|x|
// and max|w| as fp32 (non-negative floats order like their bit patterns, so
// an integer maximum is exact).  Two kernels, no atomics: kMagGroups
// workgroups each reduce a stripe to part[2 g], part[2 g + 1], then one
// workgroup reduces those.
constexpr int kMagGroups = 512;

__device__ __forceinline__ uint32_t mag_of_bf16(uint32_t b) { return (b & 0x7fffu) << 16; }

__device__ __forceinline__ uint32_t mag_of_pair(uint32_t v) { return max(mag_of_bf16(v), mag_of_bf16(v >> 16)); }

// maximum of v over the workgroup (256 threads), in every thread
__device__ __forceinline__ uint32_t wg_max(uint32_t v, uint32_t *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = max(max(red[0], red[1]), max(red[2], red[3]));
    __syncthreads();
    return v;
}

__global__ __launch_bounds__(256)
void wino_mag_kernel(const uint16_t *__restrict__ x, int64_t nx, const uint16_t *__restrict__ w, int64_t nw,
                     uint32_t *__restrict__ part) {
    __shared__ uint32_t red[4];
    uint32_t mx = 0, mw = 0;
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x, nt = (int64_t)gridDim.x * 256;
    if (((uintptr_t)x & 15) == 0) {
        // 16 bytes a lane, four loads in flight, then the elements past the last whole group of 8
        const uint4 *x8 = reinterpret_cast<const uint4 *>(x);
        const int64_t n8 = nx / 8;
        int64_t i = tid;
        for (; i + 3 * nt < n8; i += 4 * nt) {
            uint4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = x8[i + k * nt];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                mx = max(mx, max(max(mag_of_pair(v[k].x), mag_of_pair(v[k].y)),
                                 max(mag_of_pair(v[k].z), mag_of_pair(v[k].w))));
        }
        for (; i < n8; i += nt) {
            const uint4 v = x8[i];
            mx = max(mx, max(max(mag_of_pair(v.x), mag_of_pair(v.y)), max(mag_of_pair(v.z), mag_of_pair(v.w))));
        }
        for (int64_t j = 8 * n8 + tid; j < nx; j += nt) mx = max(mx, mag_of_bf16(x[j]));
    } else {
        for (int64_t j = tid; j < nx; j += nt) mx = max(mx, mag_of_bf16(x[j]));
    }
    for (int64_t j = tid; j < nw; j += nt) mw = max(mw, mag_of_bf16(w[j]));
    mx = wg_max(mx, red);
    mw = wg_max(mw, red);
    if (threadIdx.x == 0) {
        part[2 * blockIdx.x] = mx;
        part[2 * blockIdx.x + 1] = mw;
    }
}

__global__ __launch_bounds__(256)
void wino_mag_final_kernel(const uint32_t *__restrict__ part, uint32_t *__restrict__ mag) {
    __shared__ uint32_t red[4];
    uint32_t mx = 0, mw = 0;
    for (int g = threadIdx.x; g < kMagGroups; g += 256) {
        mx = max(mx, part[2 * g]);
        mw = max(mw, part[2 * g + 1]);
    }
    mx = wg_max(mx, red);
    mw = wg_max(mw, red);
    if (threadIdx.x == 0) {
        mag[0] = mx;
        mag[1] = mw;
    }
}

// 2^k with max * 2^k * 4 <= 2^13: k = 11 - E for max = m 2^E, m in [0.5, 1);
// 0 for a zero, infinite or NaN maximum (nothing to scale, or nothing that
// scaling could save).
__device__ __forceinline__ int wino_scale_exp(uint32_t magbits) {
    const float m = __uint_as_float(magbits);
    if (!(m > 0.f) || !(m <= 3.0e38f)) return 0;
    int e;
    (void)frexpf(m, &e);
    return 11 - e;
}

// 1. U: one thread per (k, c).
__global__ __launch_bounds__(256)
void wino_weight_kernel(const uint16_t *__restrict__ w, uint16_t *__restrict__ U, int Co, int C,
                        const uint32_t *__restrict__ mag) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)Co * C) return;
    const int kw = wino_scale_exp(mag[1]);
    const uint16_t *g = w + e * 9;
    float gv[3][3];
#pragma unroll
    for (int i = 0; i < 9; ++i) gv[i / 3][i % 3] = ldexpf(bf16_to_f32(g[i]), kw);
    // t = G g (4x3), u = t G^T (4x4)
    float t[4][3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        t[0][j] = gv[0][j];
        t[1][j] = 0.5f * (gv[0][j] + gv[1][j] + gv[2][j]);
        t[2][j] = 0.5f * (gv[0][j] - gv[1][j] + gv[2][j]);
        t[3][j] = gv[2][j];
    }
    const int64_t plane = (int64_t)Co * C;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float u0 = t[i][0];
        const float u1 = 0.5f * (t[i][0] + t[i][1] + t[i][2]);
        const float u2 = 0.5f * (t[i][0] - t[i][1] + t[i][2]);
        const float u3 = t[i][2];
        U[(4 * i + 0) * plane + e] = f16_bits(u0);
        U[(4 * i + 1) * plane + e] = f16_bits(u1);
        U[(4 * i + 2) * plane + e] = f16_bits(u2);
        U[(4 * i + 3) * plane + e] = f16_bits(u3);
    }
}

// 2. V: one thread per (block t, 8 consecutive channels); 16 stores of 16 bytes.
__global__ __launch_bounds__(256)
void wino_input_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ V, int C, int H, int W, int p, int TH,
                       int TW, int64_t T, const uint32_t *__restrict__ mag) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int cgrp = C / 8;
    if (e >= T * cgrp) return;
    const int kx = wino_scale_exp(mag[0]);
    const int64_t t = e / cgrp;
    const int c0 = (int)(e - t * cgrp) * 8;
    const int bw = (int)(t % TW);
    const int bh = (int)((t / TW) % TH);
    const int64_t n = t / ((int64_t)TW * TH);
    const int64_t HW = (int64_t)H * W;
    const int ih0 = 2 * bh - p, iw0 = 2 * bw - p;
    uint32_t out[16][4];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + ((int64_t)n * C + c0 + cc) * HW, (uint32_t)(HW * 2));
        float d[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ih = ih0 + i, iw = iw0 + j;
                const bool in = 0 <= ih && ih < H && 0 <= iw && iw < W;
                d[i][j] = ldexpf(bf16_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                                     xr, (int)(in ? (uint32_t)(ih * W + iw) * 2u : kOob), 0, 0)),
                                 kx);
            }
        // s = B^T d, v = s B
        float s[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[0][j] = d[0][j] - d[2][j];
            s[1][j] = d[1][j] + d[2][j];
            s[2][j] = d[2][j] - d[1][j];
            s[3][j] = d[1][j] - d[3][j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v[4] = {s[i][0] - s[i][2], s[i][1] + s[i][2], s[i][2] - s[i][1], s[i][1] - s[i][3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t h = f16_bits(v[j]);
                uint32_t &slot = out[4 * i + j][cc >> 1];
                slot = (cc & 1) ? (slot | (h << 16)) : h;
            }
        }
    }
#pragma unroll
    for (int xi = 0; xi < 16; ++xi)
        *reinterpret_cast<uint4 *>(V + (((int64_t)xi * ((C + 31) / 32) + c0 / 32) * T + t) * 32 + (c0 & 31)) =
            make_uint4(out[xi][0], out[xi][1], out[xi][2], out[xi][3]);
}

// 2'. V for C_in % 32 == 0 and W % 8 == 0: a workgroup takes 32 channels x
// 32 consecutive blocks of one block row (input rows 2bh - p .. +3).
//   Copy: the 4 input rows of the 32 channels go to LDS in aligned 16-byte
//   units (8 pixels, wholly inside or outside the image since W % 8 == 0;
//   outside ones, and rows outside the image, read as zeros): [c][row][80 px].
//   Transform: lane b on block b, four channels per thread; the 4 x 4 input
//   block of block b starts 2b pixels into the copied rows.
//   Store: each thread writes its 4 channels (8 bytes) of every xi; the 8
//   threads of a block fill its 64-byte row of the channel tile, and a tile's
//   blocks are consecutive rows.
constexpr int kWiC = 32, kWiB = 32;       // channels, blocks per workgroup
constexpr int kWiRow = 80;                // pixels per copied row (10 units)

__global__ __launch_bounds__(256)
void wino_input_tile_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ V, int C, int H, int W, int p,
                            int TH, int TW, int64_t T, int nbw, const uint32_t *__restrict__ mag) {
    __shared__ __align__(16) uint16_t Xs[kWiC * 4 * kWiRow];
    const int tid = threadIdx.x;
    const int kx = wino_scale_exp(mag[0]);
    const int c0 = blockIdx.x * kWiC;
    int r = blockIdx.y;
    const int bwg = r % nbw;
    r /= nbw;
    const int bh = r % TH;
    const int n = r / TH;
    const int bw0 = bwg * kWiB;
    const int cs = 2 * bw0 - p;                            // first input column of the tile
    const int a0 = (cs >= 0 ? cs / 8 : -((7 - cs) / 8)) * 8;   // aligned start (floor)
    const int64_t HW = (int64_t)H * W;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + ((int64_t)n * C + c0) * HW, (uint32_t)(kWiC * HW * 2));
    // copy: unit u -> (channel, row, 8-pixel unit k), k fastest
    for (int u = tid; u < kWiC * 4 * (kWiRow / 8); u += 256) {
        const int k = u % (kWiRow / 8), cr = u / (kWiRow / 8);
        const int i = cr & 3, c = cr >> 2;
        const int ih = 2 * bh - p + i, iw = a0 + 8 * k;
        const bool in = 0 <= ih && ih < H && 0 <= iw && iw < W;
        const uint4 v = bload16(xr, in ? (uint32_t)((c * HW + (int64_t)ih * W + iw) * 2) : kOob, 0);
        *reinterpret_cast<uint4 *>(&Xs[(c * 4 + i) * kWiRow + 8 * k]) = v;
    }
    __syncthreads();
    // transform: thread (block b, channels 4q .. 4q+3)
    {
        const int b = tid & 31, q = tid >> 5;
        const int col0 = cs - a0 + 2 * b;
        uint32_t out[16][2];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int c = 4 * q + cc;
            float d[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) d[i][j] = ldexpf(bf16_to_f32(Xs[(c * 4 + i) * kWiRow + col0 + j]), kx);
            float s4[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s4[0][j] = d[0][j] - d[2][j];
                s4[1][j] = d[1][j] + d[2][j];
                s4[2][j] = d[2][j] - d[1][j];
                s4[3][j] = d[1][j] - d[3][j];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v[4] = {s4[i][0] - s4[i][2], s4[i][1] + s4[i][2], s4[i][2] - s4[i][1], s4[i][1] - s4[i][3]};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t h = f16_bits(v[j]);
                    uint32_t &slot = out[4 * i + j][cc >> 1];
                    slot = (cc & 1) ? (slot | (h << 16)) : h;
                }
            }
        }
        if (bw0 + b < TW) {
            const int64_t CT = C / 32;
            const int64_t t = ((int64_t)n * TH + bh) * TW + bw0 + b;
            uint16_t *dst = V + ((int64_t)blockIdx.x * T + t) * 32 + 4 * q;    // xi = 0, channel tile c0 / 32
#pragma unroll
            for (int xi = 0; xi < 16; ++xi)
                *reinterpret_cast<uint2 *>(dst + (int64_t)xi * CT * T * 32) = make_uint2(out[xi][0], out[xi][1]);
        }
    }
}

// 3. 16 GEMMs + output transform.  LDS holds the 16 x 32 x 32 fp32 results
// (64 KB; reads run along blocks, conflict-free).
__global__ __launch_bounds__(256)
void wino_gemm_kernel(const uint16_t *__restrict__ U, const uint16_t *__restrict__ V, const float *__restrict__ bias,
                      float *__restrict__ y, Shape sh, int TH, int TW, int64_t T, int nkt, int remap,
                      const uint32_t *__restrict__ mag) {
    __shared__ float Ms[16][32][32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int unscale = -(wino_scale_exp(mag[0]) + wino_scale_exp(mag[1]));
    const int C = sh.C, Co = sh.Co;
    // block -> (channel tile, block tile): the channel tiles of one block tile
    // are consecutive logical tiles, and with remap each XCD (block % 8) runs a
    // contiguous range of them, so V's rows for a block tile come from one L2
    int64_t L = blockIdx.x;
    if (remap) L = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int k0 = (int)(L % nkt) * 32;
    const int64_t t0 = (L / nkt) * 32;
    const int64_t plane = (int64_t)Co * C;
    // A: U[xi][k0 + lane%32][c + 8*(lane/32)], B: V[xi][c/32][t0 + lane%32][c%32 + 8*(lane/32)]
    const int kr = k0 + (lane & 31);
    const int64_t tr = t0 + (lane & 31);
    const int coff = 8 * (lane >> 5);
    const __amdgpu_buffer_rsrc_t ur = make_rsrc(U, (uint32_t)(16 * plane * 2));
    const int CT = (C + 31) / 32;
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(V, (uint32_t)(16 * CT * T * 64));
    uint32_t ao[4], bo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int xi = 4 * wave + q;
        ao[q] = kr < Co ? (uint32_t)(((int64_t)xi * plane + (int64_t)kr * C + coff) * 2) : kOob;
        bo[q] = tr < T ? (uint32_t)((((int64_t)xi * CT * T + tr) * 32 + coff) * 2) : kOob;
    }
    f32x16_t acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;

    uint4 a[4], b[4], an[4], bn[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        a[q] = bload16(ur, ao[q], 0);
        b[q] = bload16(vr, bo[q], 0);
    }
    const int nst = C / 16;
    for (int st = 0; st < nst; ++st) {
        if (st + 1 < nst) {
            const uint32_t so = (uint32_t)(st + 1) * 32u;   // U: 16 channels = 32 bytes
            const uint32_t vso = (uint32_t)(((st + 1) >> 1) * T * 64 + ((st + 1) & 1) * 32);   // V: tile, half
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                an[q] = bload16(ur, ao[q] == kOob ? kOob : ao[q] + so, 0);
                bn[q] = bload16(vr, bo[q] == kOob ? kOob : bo[q] + vso, 0);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = mfma32x32x16_f16(a[q], b[q], acc[q]);
        if (st + 1 < nst) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a[q] = an[q];
                b[q] = bn[q];
            }
        }
    }
    // results to LDS: Ms[xi][k - k0][t - t0]
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) Ms[4 * wave + q][mfma32_row(r, lane)][lane & 31] = acc[q][r];
    __syncthreads();

    // output transform: Y = A^T M A for 4 (k, block) pairs per thread
    const int Ho = sh.Ho, Wo = sh.Wo;
    const int64_t oplane = (int64_t)Ho * Wo;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int pair = tid + 256 * u;
        const int kl = pair >> 5, tl = pair & 31;
        const int k = k0 + kl;
        const int64_t t = t0 + tl;
        if (k >= Co || t >= T) continue;
        float m[16];
#pragma unroll
        for (int xi = 0; xi < 16; ++xi) m[xi] = Ms[xi][kl][tl];
        // r = A^T M (2x4), then Y = r A (2x2)
        float r[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r[0][j] = m[j] + m[4 + j] + m[8 + j];
            r[1][j] = m[4 + j] - m[8 + j] - m[12 + j];
        }
        const int bw = (int)(t % TW), bh = (int)((t / TW) % TH);
        const int64_t n = t / ((int64_t)TW * TH);
        const float bv = bias ? bias[k] : 0.f;
        const int64_t yb = ((int64_t)n * Co + k) * oplane;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float y0 = ldexpf(r[i][0] + r[i][1] + r[i][2], unscale);
            const float y1 = ldexpf(r[i][1] - r[i][2] - r[i][3], unscale);
            const int oh = 2 * bh + i, ow = 2 * bw;
            if (oh >= Ho) continue;
            store_out(y, yb + (int64_t)oh * Wo + ow, y0 + bv, sh.out_bf16, sh.relu);
            if (ow + 1 < Wo) store_out(y, yb + (int64_t)oh * Wo + ow + 1, y1 + bv, sh.out_bf16, sh.relu);
        }
    }
}

struct WinoGeom {
    int TH, TW;
    int64_t T;
    size_t u_bytes, v_bytes;
    static constexpr size_t kMagBytes = 256 + 8 * kMagGroups;   // the two magnitudes, then the partial maxima
};

WinoGeom wino_geom(const Shape &sh) {
    WinoGeom g;
    g.TH = (sh.Ho + 1) / 2;
    g.TW = (sh.Wo + 1) / 2;
    g.T = (int64_t)sh.N * g.TH * g.TW;
    g.u_bytes = ((size_t)16 * sh.Co * sh.C * 2 + 255) / 256 * 256;
    g.v_bytes = (size_t)16 * g.T * ((sh.C + 31) / 32) * 64;
    return g;
}

}  // namespace

bool winograd_supported(const Shape &sh) {
    if (!(sh.ndim == 2 && sh.K == 3 && sh.s == 1 && sh.dil == 1 && sh.G == 1 && !sh.nhwc && sh.C % 16 == 0))
        return false;
    const WinoGeom g = wino_geom(sh);
    // 32-bit buffer offsets into U and V; the GEMM grid (256 threads a block) below 2^32 threads
    return (int64_t)16 * sh.Co * sh.C * 2 < (INT64_C(1) << 31) &&
           (int64_t)16 * g.T * ((sh.C + 31) / 32) * 64 < (INT64_C(1) << 31) &&
           (int64_t)((sh.Co + 31) / 32) * ((g.T + 31) / 32) < (INT64_C(1) << 24);
}

size_t winograd_workspace_bytes(const Shape &sh) {
    const WinoGeom g = wino_geom(sh);
    return g.u_bytes + g.v_bytes + WinoGeom::kMagBytes;
}

hipError_t launch_winograd_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias, float *y,
                                void *ws, hipStream_t st) {
    const WinoGeom g = wino_geom(sh);
    uint16_t *U = (uint16_t *)ws;
    uint16_t *V = (uint16_t *)((char *)ws + g.u_bytes);
    uint32_t *mag = (uint32_t *)((char *)ws + g.u_bytes + g.v_bytes);
    const int64_t nu = (int64_t)sh.Co * sh.C;
    uint32_t *part = mag + 64;
    hipLaunchKernelGGL(wino_mag_kernel, dim3(kMagGroups), dim3(256), 0, st, x, sh.x_elems(), w, sh.w_elems(), part);
    hipLaunchKernelGGL(wino_mag_final_kernel, dim3(1), dim3(256), 0, st, (const uint32_t *)part, mag);
    hipLaunchKernelGGL(wino_weight_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, st, w, U, sh.Co, sh.C,
                       (const uint32_t *)mag);
    if (sh.C % kWiC == 0 && sh.W % 8 == 0) {
        const int nbw = (g.TW + kWiB - 1) / kWiB;
        dim3 gi((unsigned)(sh.C / kWiC), (unsigned)((int64_t)sh.N * g.TH * nbw));
        hipLaunchKernelGGL(wino_input_tile_kernel, gi, dim3(256), 0, st, x, V, sh.C, sh.H, sh.W, sh.p, g.TH, g.TW, g.T,
                           nbw, (const uint32_t *)mag);
    } else {
        const int64_t nv = g.T * (sh.C / 8);
        hipLaunchKernelGGL(wino_input_kernel, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, st, x, V, sh.C, sh.H,
                           sh.W, sh.p, g.TH, g.TW, g.T, (const uint32_t *)mag);
    }
    const int nkt = (sh.Co + 31) / 32;
    const int64_t nblk = (int64_t)nkt * ((g.T + 31) / 32);
    hipLaunchKernelGGL(wino_gemm_kernel, dim3((unsigned)nblk), dim3(256), 0, st, U, V, bias, y, sh, g.TH, g.TW, g.T, nkt,
                       nblk % 8 == 0 ? 1 : 0, (const uint32_t *)mag);
    return hipGetLastError();
}

}  // namespace convfwd
