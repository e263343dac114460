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
//  2. V[xi][t][c] = (B^T d[c][t] B)[xi], fp16, for every 2x2 output block t
//     (its 4x4 input block d, zero outside the image);
//  3. for each of the 16 transform points xi the GEMM M[xi] = U[xi] @ V[xi]^T
//     (C_out x blocks, reduction over C_in) on v_mfma_f32_32x32x16_f16 with
//     fp32 accumulation, then, in the same workgroup, Y = A^T M A per block,
//     + bias, stored into y (NCHW, fp32 or bf16, optional ReLU), the last
//     block row/column cropped.
// fp16 rather than bf16 for U and V: the transformed operands are rounded
// before the products, and fp16's 11-bit significand keeps that error near
// 2^-11 of the transform-domain magnitudes (bf16's 8 bits would be 8x worse,
// the low-precision risk the page warns about).  N(0,1)-scale activations and
// weights stay far inside fp16's range.
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

// 1. U: one thread per (k, c).
__global__ __launch_bounds__(256)
void wino_weight_kernel(const uint16_t *__restrict__ w, uint16_t *__restrict__ U, int Co, int C) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)Co * C) return;
    const uint16_t *g = w + e * 9;
    float gv[3][3];
#pragma unroll
    for (int i = 0; i < 9; ++i) gv[i / 3][i % 3] = bf16_to_f32(g[i]);
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
                       int TW, int64_t T) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int cgrp = C / 8;
    if (e >= T * cgrp) return;
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
                d[i][j] = bf16_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                    xr, (int)(in ? (uint32_t)(ih * W + iw) * 2u : kOob), 0, 0));
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
        *reinterpret_cast<uint4 *>(V + ((int64_t)xi * T + t) * C + c0) =
            make_uint4(out[xi][0], out[xi][1], out[xi][2], out[xi][3]);
}

// 3. 16 GEMMs + output transform.  LDS holds the 16 x 32 x 32 fp32 results
// (64 KB; reads run along blocks, conflict-free).
__global__ __launch_bounds__(256)
void wino_gemm_kernel(const uint16_t *__restrict__ U, const uint16_t *__restrict__ V, const float *__restrict__ bias,
                      float *__restrict__ y, Shape sh, int TH, int TW, int64_t T) {
    __shared__ float Ms[16][32][32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int C = sh.C, Co = sh.Co;
    const int k0 = blockIdx.x * 32;
    const int64_t t0 = (int64_t)blockIdx.y * 32;
    const int64_t plane = (int64_t)Co * C;
    // A: U[xi][k0 + lane%32][c + 8*(lane/32)], B: V[xi][t0 + lane%32][c + 8*(lane/32)]
    const int kr = k0 + (lane & 31);
    const int64_t tr = t0 + (lane & 31);
    const int coff = 8 * (lane >> 5);
    const __amdgpu_buffer_rsrc_t ur = make_rsrc(U, (uint32_t)(16 * plane * 2));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(V, (uint32_t)(16 * T * C * 2));
    uint32_t ao[4], bo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int xi = 4 * wave + q;
        ao[q] = kr < Co ? (uint32_t)(((int64_t)xi * plane + (int64_t)kr * C + coff) * 2) : kOob;
        bo[q] = tr < T ? (uint32_t)((((int64_t)xi * T + tr) * C + coff) * 2) : kOob;
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
            const uint32_t so = (uint32_t)(st + 1) * 32u;   // 16 channels = 32 bytes
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                an[q] = bload16(ur, ao[q] == kOob ? kOob : ao[q] + so, 0);
                bn[q] = bload16(vr, bo[q] == kOob ? kOob : bo[q] + so, 0);
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
            const float y0 = r[i][0] + r[i][1] + r[i][2];
            const float y1 = r[i][1] - r[i][2] - r[i][3];
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
};

WinoGeom wino_geom(const Shape &sh) {
    WinoGeom g;
    g.TH = (sh.Ho + 1) / 2;
    g.TW = (sh.Wo + 1) / 2;
    g.T = (int64_t)sh.N * g.TH * g.TW;
    g.u_bytes = ((size_t)16 * sh.Co * sh.C * 2 + 255) / 256 * 256;
    g.v_bytes = (size_t)16 * g.T * sh.C * 2;
    return g;
}

}  // namespace

bool winograd_supported(const Shape &sh) {
    if (!(sh.ndim == 2 && sh.K == 3 && sh.s == 1 && sh.dil == 1 && sh.G == 1 && !sh.nhwc && sh.C % 16 == 0))
        return false;
    const WinoGeom g = wino_geom(sh);
    // 32-bit buffer offsets into U and V; grid y below 2^31
    return (int64_t)16 * sh.Co * sh.C * 2 < (INT64_C(1) << 31) && (int64_t)16 * g.T * sh.C * 2 < (INT64_C(1) << 31);
}

size_t winograd_workspace_bytes(const Shape &sh) {
    const WinoGeom g = wino_geom(sh);
    return g.u_bytes + g.v_bytes;
}

hipError_t launch_winograd_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias, float *y,
                                void *ws, hipStream_t st) {
    const WinoGeom g = wino_geom(sh);
    uint16_t *U = (uint16_t *)ws;
    uint16_t *V = (uint16_t *)((char *)ws + g.u_bytes);
    const int64_t nu = (int64_t)sh.Co * sh.C;
    hipLaunchKernelGGL(wino_weight_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, st, w, U, sh.Co, sh.C);
    const int64_t nv = g.T * (sh.C / 8);
    hipLaunchKernelGGL(wino_input_kernel, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, st, x, V, sh.C, sh.H, sh.W,
                       sh.p, g.TH, g.TW, g.T);
    dim3 grid((unsigned)((sh.Co + 31) / 32), (unsigned)((g.T + 31) / 32));
    hipLaunchKernelGGL(wino_gemm_kernel, grid, dim3(256), 0, st, U, V, bias, y, sh, g.TH, g.TW, g.T);
    return hipGetLastError();
}

}  // namespace convfwd
