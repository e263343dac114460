// k_depthwise.hip -- 2D convolution with one input channel per group (C_in/G
// == 1): the depthwise layer (G = C_in, "PyTorch tensor products and
// conv2d/conv3d dimension semantics", 4.3; "Conv2d from the official docs",
// 3.4), with a channel multiplier M = C_out/C_in >= 1, any K, stride, pad and
// dilation.  Output channel c*M + m reads input channel c only.
//
// There is no reduction over channels, so the matrix cores have nothing to
// contract (a K*K-long dot product per output): the layer is bound by HBM --
// each input element read once (2 or 4 bytes) and each output written once
// (4 bytes) -- and runs on the vector ALUs.  The pages make the same point
// ("Why use matrix multiplication for convolution", 4.2; tensor-semantics
// page, 4.3).
//
// A workgroup owns one input channel c of one image and a tile of TH x TW
// output positions.  It stages the input patch the tile needs -- (TH-1)*s +
// d(K-1) + 1 rows by (TW-1)*s + d(K-1) + 1 columns, zero outside the input
// (padding by bounds checks) -- in LDS as fp32, each row loaded by one wave
// with consecutive lanes on consecutive columns.  Then for each of the M
// output channels of c it computes the tile: a thread owns one output column
// and RB consecutive output rows, reads its taps from LDS and the K*K weights
// of the channel (the same for the whole workgroup) through the scalar cache,
// and stores RB fp32 values, consecutive lanes on consecutive columns.
#include "conv_internal.h"
#include "mfma_common.h"

namespace convfwd {
namespace {

constexpr int kThreads = 256;
constexpr int kRB = 4;                       // output rows per thread
constexpr int kMaxPatch = 12 * 1024;         // fp32 patch elements in LDS (48 KB)

template <typename T> __device__ __forceinline__ float ldv(const T *p, int64_t i);
template <> __device__ __forceinline__ float ldv<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldv<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
}

struct DwGeom {
    int TW, TH;          // output tile
    int PR, PC;          // patch rows / columns
    int tiles_w, tiles_h;
};

__host__ __device__ inline DwGeom dw_geom(const Shape &sh) {
    DwGeom g;
    g.TW = sh.Wo > 32 ? 64 : 32;
    g.TH = (kThreads / g.TW) * kRB;
    g.PR = (g.TH - 1) * sh.s + (sh.K - 1) * sh.dil + 1;
    g.PC = (g.TW - 1) * sh.s + (sh.K - 1) * sh.dil + 1;
    g.tiles_w = (sh.Wo + g.TW - 1) / g.TW;
    g.tiles_h = (sh.Ho + g.TH - 1) / g.TH;
    return g;
}

// KS: compile-time kernel size (0 = runtime sh.K).
template <typename T, int KS>
__global__ __launch_bounds__(kThreads)
void depthwise_kernel(Shape sh, DwGeom g, const T *__restrict__ x, const T *__restrict__ w,
                      const float *__restrict__ bias, float *__restrict__ y) {
    extern __shared__ float patch[];
    const int K = KS ? KS : sh.K;
    const int M = sh.Co / sh.C;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // blockIdx.x -> (plane = n*C + c, tile row, tile column), tile column fastest
    int64_t b = blockIdx.x;
    const int tw = (int)(b % g.tiles_w); b /= g.tiles_w;
    const int th = (int)(b % g.tiles_h); b /= g.tiles_h;
    const int64_t plane = b;                              // n*C + c
    const int c = (int)(plane % sh.C);
    const int64_t n = plane / sh.C;
    const int oh0 = th * g.TH, ow0 = tw * g.TW;
    const int ih0 = oh0 * sh.s - sh.p, iw0 = ow0 * sh.s - sh.p;

    // stage the patch: wave w loads rows w, w+4, ...
    const T *xp = x + plane * ((int64_t)sh.H * sh.W);
    for (int r = wave; r < g.PR; r += kThreads / 64) {
        const int ih = ih0 + r;
        const bool rin = 0 <= ih && ih < sh.H;
        for (int cc = lane; cc < g.PC; cc += 64) {
            const int iw = iw0 + cc;
            float v = 0.f;
            if (rin && 0 <= iw && iw < sh.W) v = ldv(xp, (int64_t)ih * sh.W + iw);
            patch[r * g.PC + cc] = v;
        }
    }
    __syncthreads();

    const int col = tid % g.TW, strip = tid / g.TW;
    const int ow = ow0 + col;
    const int ohs = oh0 + strip * kRB;
    if (ow >= sh.Wo || ohs >= sh.Ho) return;              // no barrier below
    const float *pb = patch + (strip * kRB * sh.s) * g.PC + col * sh.s;
    const int64_t oplane = (int64_t)sh.Ho * sh.Wo;

    for (int m = 0; m < M; ++m) {
        const int oc = c * M + m;
        const T *wc = w + (int64_t)oc * K * K;
        const float bv = bias ? bias[oc] : 0.f;
        float acc[kRB];
#pragma unroll
        for (int r = 0; r < kRB; ++r) acc[r] = 0.f;
#pragma unroll
        for (int kh = 0; kh < K; ++kh) {
#pragma unroll
            for (int kw = 0; kw < K; ++kw) {
                const float wv = ldv(wc, kh * K + kw);
                const float *pt = pb + (kh * sh.dil) * g.PC + kw * sh.dil;
#pragma unroll
                for (int r = 0; r < kRB; ++r) acc[r] = __builtin_fmaf(pt[r * sh.s * g.PC], wv, acc[r]);
            }
        }
        float *yp = y + (n * sh.Co + oc) * oplane + (int64_t)ohs * sh.Wo + ow;
#pragma unroll
        for (int r = 0; r < kRB; ++r)
            if (ohs + r < sh.Ho) yp[(int64_t)r * sh.Wo] = acc[r] + bv;
    }
}

template <typename T>
hipError_t launch_dw(const Shape &sh, const T *x, const T *w, const float *bias, float *y, hipStream_t st) {
    const DwGeom g = dw_geom(sh);
    const int64_t blocks = (int64_t)sh.N * sh.C * g.tiles_h * g.tiles_w;
    const size_t lds = (size_t)g.PR * g.PC * sizeof(float);
    if (sh.K == 3)
        hipLaunchKernelGGL((depthwise_kernel<T, 3>), dim3((unsigned)blocks), dim3(kThreads), lds, st, sh, g, x,
                           w, bias, y);
    else
        hipLaunchKernelGGL((depthwise_kernel<T, 0>), dim3((unsigned)blocks), dim3(kThreads), lds, st, sh, g, x,
                           w, bias, y);
    return hipGetLastError();
}

}  // namespace

bool depthwise_supported(const Shape &sh) {
    if (sh.ndim != 2 || sh.Cg() != 1) return false;
    const DwGeom g = dw_geom(sh);
    if ((int64_t)g.PR * g.PC > kMaxPatch) return false;
    const int64_t blocks = (int64_t)sh.N * sh.C * g.tiles_h * g.tiles_w;
    return blocks < (INT64_C(1) << 31);
}

hipError_t launch_depthwise_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias,
                                 float *y, hipStream_t st) {
    return launch_dw<uint16_t>(sh, x, w, bias, y, st);
}

hipError_t launch_depthwise_f32(const Shape &sh, const float *x, const float *w, const float *bias, float *y,
                                hipStream_t st) {
    return launch_dw<float>(sh, x, w, bias, y, st);
}

}  // namespace convfwd
