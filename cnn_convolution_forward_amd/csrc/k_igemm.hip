// k_igemm.hip -- general bf16 MFMA GEMM  Y = W_row @ X_col  for any convolution
// shape (2D or 3D, any K, stride, pad), in two flavours that share one body:
//
//  * implicit: X_col is never stored; each K-slice of its tile is gathered from
//    x straight into LDS with bounds checks (zero padding without a padded copy)
//    and discarded after the multiply ("Why use matrix multiplication for
//    convolution", 4.3: fused im2col-GEMM; "Hand-writing Conv2D", 4.1: unfold
//    per tile and drop it after use);
//  * explicit: the same tile is read from an X_col matrix in device memory that
//    the im2col kernel wrote (the pages' two-step form, same page 2.3 and 3.2).
//
// GEMM view: M = C_out (rows of W_row), N = N*Do*Ho*Wo output pixels, K =
// C_in*K^dims in the natural OIHW order r = ((ic*Kd + kd)*K + kh)*K + kw, so a
// row of W_row is contiguous in memory.  With groups G the problem is G
// independent GEMMs of C_out/G x (C_in/G * K^dims) each, one per blockIdx.z
// ("PyTorch tensor products and conv2d/conv3d dimension semantics", 4.3); with
// dilation d the taps of the gather sit d inputs apart (same page, 4.2).  Block tile BM x 128 pixels x 32 k,
// four waves in a 2 x 2 grid, v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
// The epilogue adds bias[oc] and stores fp32 straight into N C_out (D) H W
// order: the reshape + axis swap of "Why use matrix multiplication for
// convolution", 3.2, fused into the store.
//
// A third flavour serves the data gradient of a strided convolution: the
// input it gathers is dout seen through zero insertion (ups - 1 zeros between
// neighbours, the transposed convolution), so a virtual coordinate v reads
// dout[v / ups] when v % ups == 0 and 0 otherwise.
//
// Options of the general entry point: channels-last x and y (sh.nhwc), and an
// epilogue with ReLU and/or bf16 output (sh.relu, sh.out_bf16).
//
// This is the route for every shape the specialised kernels do not cover.
#include "conv_internal.h"
#include "mfma_common.h"

namespace convfwd {
namespace {

constexpr int kBN = 128;      // pixels per block
constexpr int kBK = 32;       // k per LDS stage
constexpr int kLdk = kBK + 8; // padded k stride in LDS: 80-byte rows keep 16-byte reads conflict-free

enum { kImplicit = 0, kExplicit = 1, kUpsampled = 2 };

template <int BM, int kMode>
__global__ __launch_bounds__(256)
void igemm_generic_kernel(Shape sh, const uint16_t *__restrict__ src, const uint16_t *__restrict__ w,
                          const float *__restrict__ bias, float *__restrict__ y,
                          int64_t P, int Kg, int w_vec, int g0) {
    constexpr int MI = BM / 64;               // 32-row MFMA tiles per wave (wave covers BM/2 rows)
    __shared__ __align__(16) uint16_t As[2][BM][kLdk];
    __shared__ __align__(16) uint16_t Bs[2][kBN][kLdk];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM;               // first row of the tile inside its group
    const int64_t j0 = (int64_t)blockIdx.x * kBN;
    const int grp = g0 + (int)blockIdx.z;
    const int Cog = sh.Co / sh.G, Cg = sh.C / sh.G;
    const int oc_base = grp * Cog;                  // first output channel of the group
    const uint16_t *wg = w + (int64_t)oc_base * Kg;

    // ---- B loader: this thread owns pixel bpx of the tile and k-quads bkq, bkq+2.
    const int bpx = tid & (kBN - 1);
    const int bkq = tid >> 7;                  // wave-uniform
    const int64_t jp = j0 + bpx;
    const bool pvalid = jp < P;
    int id0 = 0, ih0 = 0, iw0 = 0;
    const uint16_t *xn = src;
    if (kMode != kExplicit && pvalid) {
        int64_t t = jp;
        int ow = (int)(t % sh.Wo); t /= sh.Wo;
        int oh = (int)(t % sh.Ho); t /= sh.Ho;
        int od = (int)(t % sh.Do); t /= sh.Do;
        // image t, first channel of the group: NCHW (channel planes) or NHWC (channel fastest)
        xn = src + (sh.nhwc ? t * sh.C * sh.in_plane() + (int64_t)grp * Cg
                            : (t * sh.C + (int64_t)grp * Cg) * sh.in_plane());
        id0 = od * sh.sd - sh.pd;
        ih0 = oh * sh.s - sh.p;
        iw0 = ow * sh.s - sh.p;
    }
    const int KK = sh.K * sh.K;
    const int taps = sh.Kd * KK;
    const int64_t HW = (int64_t)sh.H * sh.W;
    // element (ic, spatial s) of an image sits at ic * cstride + s * pstride
    const int64_t cstride = sh.nhwc ? 1 : sh.in_plane(), pstride = sh.nhwc ? sh.C : 1;

    uint4 a_reg[MI];
    uint4 b_reg[2];

    auto load_stage = [&](int k0) {
        // A: W_row[m0 + row][k0 + kq*8 .. +7], unit u = tid + 256*i -> row u/4, kq u%4.
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            int u = tid + 256 * i;
            int row = u >> 2, kq = u & 3;
            int oc = m0 + row, k = k0 + kq * 8;
            if (w_vec && oc < Cog && k < Kg) {
                a_reg[i] = *reinterpret_cast<const uint4 *>(wg + (int64_t)oc * Kg + k);
            } else {
                uint16_t v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = (oc < Cog && k + e < Kg) ? wg[(int64_t)oc * Kg + k + e] : (uint16_t)0;
                a_reg[i] = pack8(v);
            }
        }
        // B: X_col[k0 + kq*8 + e][jp] for e = 0..7.
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int kq = bkq + 2 * i;
            int k = k0 + kq * 8;
            uint16_t v[8];
            if (kMode == kExplicit) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = (pvalid && k + e < Kg) ? src[((int64_t)grp * Kg + k + e) * P + jp] : (uint16_t)0;
            } else {
                int ic = k / taps, rem = k - ic * taps;
                int kd = rem / KK; rem -= kd * KK;
                int kh = rem / sh.K, kw = rem - kh * sh.K;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint16_t val = 0;
                    if (pvalid && ic < Cg) {
                        int id = id0 + kd * sh.dild, ih = ih0 + kh * sh.dil, iw = iw0 + kw * sh.dil;
                        if (kMode == kUpsampled) {
                            // virtual coordinates over the zero-inserted input
                            const bool on = 0 <= id && id < (sh.D - 1) * sh.upsd + 1 && id % sh.upsd == 0 &&
                                            0 <= ih && ih < (sh.H - 1) * sh.ups + 1 && ih % sh.ups == 0 &&
                                            0 <= iw && iw < (sh.W - 1) * sh.ups + 1 && iw % sh.ups == 0;
                            if (on)
                                val = xn[(int64_t)ic * cstride +
                                         ((int64_t)(id / sh.upsd) * HW + (int64_t)(ih / sh.ups) * sh.W + iw / sh.ups) *
                                             pstride];
                        } else if (0 <= id && id < sh.D && 0 <= ih && ih < sh.H && 0 <= iw && iw < sh.W) {
                            val = xn[(int64_t)ic * cstride + ((int64_t)id * HW + (int64_t)ih * sh.W + iw) * pstride];
                        }
                    }
                    v[e] = val;
                    if (++kw == sh.K) { kw = 0; if (++kh == sh.K) { kh = 0; if (++kd == sh.Kd) { kd = 0; ++ic; } } }
                }
            }
            b_reg[i] = pack8(v);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            int u = tid + 256 * i;
            *reinterpret_cast<uint4 *>(&As[buf][u >> 2][(u & 3) * 8]) = a_reg[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *reinterpret_cast<uint4 *>(&Bs[buf][bpx][(bkq + 2 * i) * 8]) = b_reg[i];
    };

    f32x16_t acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (Kg + kBK - 1) / kBK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_stage((kt + 1) * kBK);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            uint4 a[MI], b[2];
            const int kof = kk * 16 + (lane >> 5) * 8;
#pragma unroll
            for (int i = 0; i < MI; ++i)
                a[i] = *reinterpret_cast<const uint4 *>(&As[buf][wm * (BM / 2) + i * 32 + (lane & 31)][kof]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const uint4 *>(&Bs[buf][wn * 64 + j * 32 + (lane & 31)][kof]);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: y[n][oc][q] (NHWC: y[n][q][oc]) = acc + bias[oc], then the
    // optional ReLU and bf16 rounding
    const int64_t plane = sh.out_plane();
    const int64_t ocs = sh.nhwc ? 1 : plane, qs = sh.nhwc ? sh.Co : 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t px = j0 + wn * 64 + j * 32 + (lane & 31);
        if (px >= P) continue;
        const int64_t n = px / plane, q = px - n * plane;
        const int64_t yb = n * sh.Co * plane + q * qs;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ocl = m0 + wm * (BM / 2) + i * 32 + mfma32_row(r, lane);
                const int oc = oc_base + ocl;
                if (ocl < Cog)
                    store_out(y, yb + (int64_t)oc * ocs, acc[i][j][r] + (bias ? bias[oc] : 0.f), sh.out_bf16,
                              sh.relu);
            }
    }
}

template <int kMode>
hipError_t launch_generic(const Shape &sh, const uint16_t *src, const uint16_t *w,
                          const float *bias, float *y, hipStream_t st) {
    const int64_t P = sh.pixels();
    const int Kg = (int)sh.kgemm();
    const int w_vec = (Kg % 8 == 0) && ((uintptr_t)w % 16 == 0);
    const unsigned gx = (unsigned)((P + kBN - 1) / kBN);
    const int Cog = sh.Co / sh.G;
    constexpr int kMaxGridZ = 65535;
    // groups beyond the grid's z limit go in further launches (g0 = first group)
    for (int g0 = 0; g0 < sh.G; g0 += kMaxGridZ) {
        const unsigned gz = (unsigned)(sh.G - g0 < kMaxGridZ ? sh.G - g0 : kMaxGridZ);
        if (Cog > 64) {
            dim3 grid(gx, (unsigned)((Cog + 127) / 128), gz);
            hipLaunchKernelGGL((igemm_generic_kernel<128, kMode>), grid, dim3(256), 0, st, sh, src, w,
                               bias, y, P, Kg, w_vec, g0);
        } else {
            dim3 grid(gx, (unsigned)((Cog + 63) / 64), gz);
            hipLaunchKernelGGL((igemm_generic_kernel<64, kMode>), grid, dim3(256), 0, st, sh, src, w,
                               bias, y, P, Kg, w_vec, g0);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_igemm_generic_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w,
                                     const float *bias, float *y, hipStream_t st) {
    return launch_generic<kImplicit>(sh, x, w, bias, y, st);
}

hipError_t launch_gemm_xcol_bf16(const Shape &sh, const uint16_t *w, const uint16_t *xcol,
                                 const float *bias, float *y, hipStream_t st) {
    return launch_generic<kExplicit>(sh, xcol, w, bias, y, st);
}

hipError_t launch_igemm_upsampled_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias,
                                       float *y, hipStream_t st) {
    return launch_generic<kUpsampled>(sh, x, w, bias, y, st);
}

}  // namespace convfwd
