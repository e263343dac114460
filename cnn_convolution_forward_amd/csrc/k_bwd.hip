// k_bwd.hip -- the backward pass's own kernels: the weight gradient on the
// matrix cores, the bias gradient, and the weight flip that turns the data
// gradient into a forward convolution.
//
// Gradients ("Hand-writing Conv2D", 5.1; "Why use matrix multiplication for
// convolution", 3.3), for y = conv(x, w) + b and upstream gradient dout:
//   db[oc]  = sum over (n, positions) of dout[n][oc];
//   dW_row  = dout_col @ X_col^T : per group g, a GEMM of C_out/G x
//             (C_in/G * K^dims) whose reduction runs over all N * H_out * W_out
//             output positions;
//   dx      = col2im(W_row^T @ dout_col) : the same as a convolution of dout
//             (zero-inserted by the stride) with the weights transposed per
//             group (C_in x C_out/G) and every tap reversed -- the flip below
//             feeds that convolution to the forward kernels.
//
// Weight gradient kernel: the reduction over positions is long and the output
// small (128 x 1152 for a 3x3, 128-channel layer), so the positions are cut
// into `splits` ranges, one workgroup per (128-column tile, channel tile,
// range, group).  Each writes its partial product to a workspace; a second
// kernel adds the partials in a fixed order, so the result is bitwise
// reproducible (no atomics).  Tiles: A = dout rows (C_out/G channels x 32
// positions per stage, contiguous along positions), B = X_col^T gathered from
// x with bounds checks (32 positions x 128 columns (ic, kd, kh, kw)), both
// staged in LDS with the reduction contiguous, v_mfma_f32_32x32x16_bf16.
// Depthwise layers (one input channel per group) have their own VALU kernel,
// and 3x3 stride-1 pad-1 layers a kernel that shares the dout operand across
// the nine taps.
#include "conv_internal.h"
#include "mfma_common.h"
#include "conv3x3_common.h"

namespace convfwd {
namespace {

constexpr int kBN = 128;      // X_col columns per tile
constexpr int kBK = 32;       // positions per LDS stage
constexpr int kLdk = kBK + 8; // 80-byte rows: 16-byte reads of 8 consecutive rows are conflict-free
constexpr int kTargetBlocks = 512;

__global__ __launch_bounds__(256)
void flip_weights_kernel(const uint16_t *__restrict__ w, uint16_t *__restrict__ wf, int Cg, int Cog, int G,
                         int taps, int64_t total) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    // e indexes w as (oc = g*Cog + ocl, j, t)
    const int t = (int)(e % taps);
    const int64_t r = e / taps;
    const int j = (int)(r % Cg);
    const int oc = (int)(r / Cg);
    const int g = oc / Cog, ocl = oc - g * Cog;
    wf[(((int64_t)g * Cg + j) * Cog + ocl) * taps + (taps - 1 - t)] = w[e];
}

// BVEC: a pointwise layer (K = 1, stride 1, pad 0, plane % 8 == 0, 16-byte
// aligned x): X_col^T is x itself, so B loads like A -- 16 bytes of 8
// consecutive positions, four lanes on one column's 32 positions.
// part_b (may be null): the bias gradient's partial sums [split][oc], added up
// by the column-tile-0 workgroups from the dout tiles already in LDS.
template <int BM, int BVEC>
__global__ __launch_bounds__(256)
void wgrad_kernel(Shape sh, const uint16_t *__restrict__ x, const uint16_t *__restrict__ dout,
                  float *__restrict__ part, float *__restrict__ part_b, int64_t P, int Kg, int64_t chunk, int splits,
                  int g0, int a_vec) {
    constexpr int MI = BM / 64;
    __shared__ __align__(16) uint16_t As[2][BM][kLdk];
    __shared__ __align__(16) uint16_t Bs[2][kBN][kLdk];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * kBN;                      // first X_col column
    const int m0 = blockIdx.y * BM;                       // first channel inside the group
    const int split = (int)blockIdx.z % splits;
    const int grp = g0 + (int)blockIdx.z / splits;
    const int Cog = sh.Co / sh.G, Cg = sh.C / sh.G;
    const int64_t k_begin = (int64_t)split * chunk;
    const int64_t k_end = k_begin + chunk < P ? k_begin + chunk : P;
    const int64_t plane = sh.out_plane();
    const int64_t HW = (int64_t)sh.H * sh.W;

    // B loader: column bj of the tile, position quads bkq and bkq + 2
    const int bj = tid & (kBN - 1), bkq = tid >> 7;
    const int jcol = n0 + bj;
    const bool jvalid = jcol < Kg;
    int ic = 0, kd = 0, kh = 0, kw = 0;
    if (jvalid) {
        const int taps = sh.Kd * sh.K * sh.K;
        ic = jcol / taps;
        int rem = jcol - ic * taps;
        kd = rem / (sh.K * sh.K);
        rem -= kd * sh.K * sh.K;
        kh = rem / sh.K;
        kw = rem - kh * sh.K;
    }
    const int dz = kd * sh.dild - sh.pd, dy = kh * sh.dil - sh.p, dxo = kw * sh.dil - sh.p;
    const uint16_t *xg = x + (int64_t)(grp * Cg + ic) * sh.in_plane();    // channel of image 0
    const int64_t img_stride = (int64_t)sh.C * sh.in_plane();
    const uint16_t *dg = dout + (int64_t)grp * Cog * plane;                // channel g*Cog of image 0
    const int64_t dimg = (int64_t)sh.Co * plane;

    uint4 a_reg[MI], b_reg[2];
    auto load_stage = [&](int64_t k0) {
        // A: dout[n][oc][q] for 8 consecutive positions of row m
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int u = tid + 256 * i;
            const int row = u >> 2, kq = u & 3;
            const int oc = m0 + row;
            const int64_t kk = k0 + kq * 8;
            if (a_vec && oc < Cog && kk + 8 <= k_end) {
                const int n = (int)kk / (int)plane, q = (int)kk - n * (int)plane;
                a_reg[i] = *reinterpret_cast<const uint4 *>(dg + n * dimg + (int64_t)oc * plane + q);
            } else {
                uint16_t v[8];
                int64_t n = (int)kk / (int)plane, q = (int)kk - n * plane;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[e] = (oc < Cog && kk + e < k_end) ? dg[n * dimg + (int64_t)oc * plane + q] : (uint16_t)0;
                    if (++q == plane) { q = 0; ++n; }
                }
                a_reg[i] = pack8(v);
            }
        }
        if (BVEC) {
            // unit u -> (column u / 4, positions 8 (u % 4) ..): ranges are
            // multiples of 32 and P of 8, so a unit is all in or all out
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int u = tid + 256 * i;
                const int jc = n0 + (u >> 2);
                const int64_t kk = k0 + (u & 3) * 8;
                if (jc < Kg && kk < k_end) {
                    const int n = (int)kk / (int)plane, q = (int)kk - n * (int)plane;
                    b_reg[i] = *reinterpret_cast<const uint4 *>(x + ((int64_t)n * sh.C + grp * Cg + jc) * plane + q);
                } else {
                    b_reg[i] = make_uint4(0, 0, 0, 0);
                }
            }
            return;
        }
        // B: x at the tap of column jcol for 8 consecutive positions
        // (32-bit position arithmetic: P = N * output positions < 2^31)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t kk = k0 + (bkq + 2 * i) * 8;
            uint16_t v[8];
            int t = (int)kk;
            int ow = t % sh.Wo; t /= sh.Wo;
            int oh = t % sh.Ho; t /= sh.Ho;
            int od = t % sh.Do;
            int64_t n = t / sh.Do;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint16_t val = 0;
                if (jvalid && kk + e < k_end) {
                    const int id = od * sh.sd + dz, ih = oh * sh.s + dy, iw = ow * sh.s + dxo;
                    if (0 <= id && id < sh.D && 0 <= ih && ih < sh.H && 0 <= iw && iw < sh.W)
                        val = xg[n * img_stride + (int64_t)id * HW + (int64_t)ih * sh.W + iw];
                }
                v[e] = val;
                if (++ow == sh.Wo) { ow = 0; if (++oh == sh.Ho) { oh = 0; if (++od == sh.Do) { od = 0; ++n; } } }
            }
            b_reg[i] = pack8(v);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int u = tid + 256 * i;
            *reinterpret_cast<uint4 *>(&As[buf][u >> 2][(u & 3) * 8]) = a_reg[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = tid + 256 * i;
            if (BVEC)
                *reinterpret_cast<uint4 *>(&Bs[buf][u >> 2][(u & 3) * 8]) = b_reg[i];
            else
                *reinterpret_cast<uint4 *>(&Bs[buf][bj][(bkq + 2 * i) * 8]) = b_reg[i];
        }
    };

    f32x16_t acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = k_end > k_begin ? (int)((k_end - k_begin + kBK - 1) / kBK) : 0;
    // bias: thread tid adds row tid / TPR of each dout tile, positions
    // (tid % TPR) * EPT .. +EPT-1 (positions past the range and rows past
    // C_out/G are zeros in the tile)
    constexpr int TPR = 256 / BM, EPT = kBK / TPR;
    const bool do_b = part_b != nullptr && blockIdx.x == 0;
    float bsum = 0.f;
    if (nk > 0) {
        load_stage(k_begin);
        store_stage(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_stage(k_begin + (int64_t)(kt + 1) * kBK);
        if (do_b) {
#pragma unroll
            for (int v = 0; v < EPT / 8; ++v) {
                const uint4 u = *reinterpret_cast<const uint4 *>(&As[buf][tid / TPR][(tid % TPR) * EPT + 8 * v]);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bsum += __uint_as_float(w4[j] << 16) + __uint_as_float(w4[j] & 0xffff0000u);
            }
        }
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

    if (do_b) {
        // the TPR partial sums of a row meet in LDS (the stage buffers are free)
        float *red = reinterpret_cast<float *>(&As[0][0][0]);
        red[tid] = bsum;
        __syncthreads();
        if (tid % TPR == 0) {
            float r = 0.f;
#pragma unroll
            for (int k = 0; k < TPR; ++k) r += red[tid + k];
            const int ocl = m0 + tid / TPR;
            if (ocl < Cog) part_b[(int64_t)split * sh.Co + grp * Cog + ocl] = r;
        }
    }
    // partial[split][oc][jcol]: 32 lanes on 32 consecutive columns
    float *pp = part + (int64_t)split * sh.Co * Kg;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (col >= Kg) continue;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ocl = m0 + wm * (BM / 2) + i * 32 + mfma32_row(r, lane);
                if (ocl < Cog) pp[(int64_t)(grp * Cog + ocl) * Kg + col] = acc[i][j][r];
            }
    }
}

// Weight gradient with one input channel per group (2D depthwise layers):
// nothing to contract across channels, so no GEMM -- one workgroup per
// (output channel, range of images) sums dout * x over its positions for all
// K*K taps on the vector ALUs (x read through buffer loads that return 0
// outside the image), reduces the taps across the workgroup in a fixed tree,
// and writes one partial per tap.
template <int KS>
__global__ __launch_bounds__(256)
void wgrad_dw_kernel(Shape sh, const uint16_t *__restrict__ x, const uint16_t *__restrict__ dout,
                     float *__restrict__ part, int splits, int imgs_per_split) {
    // KS: compile-time kernel size (0: runtime K <= 7, taps held in a 49-entry array)
    constexpr int KK = KS ? KS * KS : 49;
    __shared__ float red[256];
    const int oc = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
    const int M = sh.Co / sh.C, ic = oc / M;
    const int K = KS ? KS : sh.K, taps = K * K;
    const int64_t plane = sh.out_plane(), HW = (int64_t)sh.H * sh.W;
    const int n0 = split * imgs_per_split;
    const int n1 = n0 + imgs_per_split < sh.N ? n0 + imgs_per_split : sh.N;
    float acc[KK];
#pragma unroll
    for (int t = 0; t < KK; ++t) acc[t] = 0.f;
    // kU positions per thread per iteration, all their loads issued before the
    // FMAs use them (positions past the plane read 0 through kOob)
    constexpr int kU = KS ? 4 : 1;
    for (int n = n0; n < n1; ++n) {
        const __amdgpu_buffer_rsrc_t dr = make_rsrc(dout + ((int64_t)n * sh.Co + oc) * plane, (uint32_t)(plane * 2));
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + ((int64_t)n * sh.C + ic) * HW, (uint32_t)(HW * 2));
        // 32-bit position arithmetic: a plane is below 2^31 elements
        const int pl = (int)plane;
        for (int q0 = tid; q0 < pl; q0 += 256 * kU) {
            float g[kU], xv[kU][KK];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int q = q0 + 256 * u;
                const bool qin = q < pl;
                const int oh = q / sh.Wo, ow = q - oh * sh.Wo;
                g[u] = bf16_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                    dr, (int)(qin ? (uint32_t)q * 2u : kOob), 0, 0));
                const int ih0 = oh * sh.s - sh.p, iw0 = ow * sh.s - sh.p;
#pragma unroll
                for (int t = 0; t < KK; ++t) {
                    const int kh = t / K, kw = t - kh * K;
                    const int ih = ih0 + kh * sh.dil, iw = iw0 + kw * sh.dil;
                    const bool in = qin && t < taps && 0 <= ih && ih < sh.H && 0 <= iw && iw < sh.W;
                    const uint32_t off = in ? (uint32_t)(ih * sh.W + iw) * 2u : kOob;
                    xv[u][t] = bf16_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(xr, (int)off, 0, 0));
                }
            }
#pragma unroll
            for (int u = 0; u < kU; ++u)
#pragma unroll
                for (int t = 0; t < KK; ++t) acc[t] = __builtin_fmaf(g[u], xv[u][t], acc[t]);
        }
    }
    float *pp = part + ((int64_t)split * sh.Co + oc) * taps;
#pragma unroll
    for (int t = 0; t < KK; ++t) {
        if (t < taps) {
            red[tid] = acc[t];
            __syncthreads();
            for (int h = 128; h > 0; h >>= 1) {
                if (tid < h) red[tid] += red[tid + h];
                __syncthreads();
            }
            if (tid == 0) pp[t] = red[0];
            __syncthreads();
        }
    }
}

// The same for 3x3, stride 1, pad = dilation DL (1 or 2), W % 8 == 0, with
// 16-byte loads: a thread task is (image, 8-column group, 4 output rows DL
// apart); per output row it reads the 8 dout values with one load and the
// 8-pixel units of one new input row (the unit under them and its two
// neighbours: the DL halo columns fall there; units and rows outside the
// image read zeros), the other two input rows staying in registers from the
// rows before, then does the 72 FMAs of 9 taps x 8 positions.  One
// resource spans all of x (and of dout), below 2 GiB, so lanes of one wave
// may sit in different images.  The 9 tap sums of the 256 threads meet in
// one fixed tree in LDS.
template <int DL>
__global__ __launch_bounds__(256)
void wgrad_dw3_kernel(Shape sh, const uint16_t *__restrict__ x, const uint16_t *__restrict__ dout,
                      float *__restrict__ part, float *__restrict__ part_b, int imgs_per_split) {
    // part_b (may be null): the bias gradient's partial sums [split][oc],
    // from the same dout loads
    __shared__ float red[10][256];
    const int oc = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
    const int M = sh.Co / sh.C, ic = oc / M;
    const int H = sh.H, W = sh.W, G8 = W / 8;
    const uint32_t HW = (uint32_t)H * (uint32_t)W;
    const int n0 = split * imgs_per_split;
    const int n1 = n0 + imgs_per_split < sh.N ? n0 + imgs_per_split : sh.N;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)sh.N * sh.C * HW * 2));
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dout, (uint32_t)((int64_t)sh.N * sh.Co * HW * 2));
    float acc[10];                     // 9 taps, then the bias
#pragma unroll
    for (int t = 0; t < 10; ++t) acc[t] = 0.f;
    // task = (image, column group, band of kRB output rows DL apart): rows
    // oh0 + DL*i, i < kRB, with oh0 = band*DL*kRB + phase.  The three input
    // rows under output row oh are oh - DL, oh, oh + DL, so the window slides
    // by one row per output row: kRB + 2 rows of 3 units a task.
    constexpr int kRB = 4;
    const int bands = (H + DL * kRB - 1) / (DL * kRB);
    const int per_img = G8 * bands * DL;
    const int tasks = (n1 - n0) * per_img;
    auto load_row = [&](uint32_t xb, int ih, int cg, uint4 (&u3)[3]) {
        const bool rin = 0 <= ih && ih < H;
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int cu = cg - 1 + u;
            const bool in = rin && 0 <= cu && cu < G8;
            u3[u] = bload16(xr, in ? (xb + (uint32_t)ih * W + 8 * cu) * 2 : kOob, 0);
        }
    };
    auto unpack24 = [](const uint4 (&u3)[3], float (&xs)[24]) {
        const uint32_t w12[12] = {u3[0].x, u3[0].y, u3[0].z, u3[0].w, u3[1].x, u3[1].y,
                                  u3[1].z, u3[1].w, u3[2].x, u3[2].y, u3[2].z, u3[2].w};
#pragma unroll
        for (int j = 0; j < 12; ++j) {
            xs[2 * j] = __uint_as_float(w12[j] << 16);
            xs[2 * j + 1] = __uint_as_float(w12[j] & 0xffff0000u);
        }
    };
    for (int task = tid; task < tasks; task += 256) {
        const int nn = task / per_img;
        int r = task - nn * per_img;
        const int cg = r % G8;
        r /= G8;
        const int phase = r % DL, band = r / DL;
        const int oh0 = band * DL * kRB + phase;
        const uint32_t n = (uint32_t)(n0 + nn);
        const uint32_t xb = (n * sh.C + ic) * HW;
        const uint32_t db = (n * sh.Co + oc) * HW + 8 * cg;
        uint4 wa[3], wb[3], wc[3];
        load_row(xb, oh0 - DL, cg, wa);
        load_row(xb, oh0, cg, wb);
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
            const int oh = oh0 + DL * i;
            load_row(xb, oh + DL, cg, wc);
            const uint4 dv = bload16(dr, oh < H ? (db + (uint32_t)oh * W) * 2 : kOob, 0);
            float d[8];
            {
                const uint32_t w4[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    d[2 * j] = __uint_as_float(w4[j] << 16);
                    d[2 * j + 1] = __uint_as_float(w4[j] & 0xffff0000u);
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[9] += d[j];
            // tap (kh, kw) at output column 8cg + j reads input column 8cg + j + (kw - 1) DL,
            // element 8 + j + (kw - 1) DL of the three units of input row oh + (kh - 1) DL
#pragma unroll
            for (int kh = 0; kh < 3; ++kh) {
                float xs[24];
                unpack24(kh == 0 ? wa : kh == 1 ? wb : wc, xs);
#pragma unroll
                for (int kw = 0; kw < 3; ++kw)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[kh * 3 + kw] = __builtin_fmaf(d[j], xs[8 + j + (kw - 1) * DL], acc[kh * 3 + kw]);
            }
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                wa[u] = wb[u];
                wb[u] = wc[u];
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 10; ++t) red[t][tid] = acc[t];
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (tid < h) {
#pragma unroll
            for (int t = 0; t < 10; ++t) red[t][tid] += red[t][tid + h];
        }
        __syncthreads();
    }
    if (tid < 9) part[((int64_t)split * sh.Co + oc) * 9 + tid] = red[tid][0];
    if (tid == 9 && part_b) part_b[(int64_t)split * sh.Co + oc] = red[9][0];
}

constexpr int kDwMaxTaps = 49;   // K <= 7

bool wgrad_dw_ok(const Shape &sh) {
    return sh.ndim == 2 && sh.Cg() == 1 && sh.K * sh.K <= kDwMaxTaps && (int64_t)sh.H * sh.W * 2 < (INT64_C(1) << 31) &&
           sh.out_plane() * 2 < (INT64_C(1) << 31);
}

// Weight gradient of a 3x3, stride-1 layer with pad = dilation (1 or 2):
// NCHW, W % 8 == 0, W <= 64, C_in and C_out multiples of 64.  The nine taps
// share one operand: for tap (kh, kw), dW[:, :, kh, kw] = dout_mat (C_out x
// positions) @ x_shift(kh, kw)^T.  A workgroup (64 output x 64 input
// channels; four waves (wm, wn) of 32 x 32 per tap, 9 accumulator tiles)
// runs over a range of output rows, one row (n, oh) a stage.  The stage's
// operands are copied into LDS by coalesced direct-to-LDS loads of 16-byte
// units of contiguous rows (read straight from global memory, with 32
// channel planes per load instruction, they kept the vector-memory pipeline
// busy with cache-line lookups at ~11% of the MFMA peak):
//   dout [oc 64][DU units]: the row's W/8 units, then zeros up to 16 x
//        ceil(W/16) positions (DU odd, so 8 rows hit 8 bank groups);
//   x    [ic 64][kh 3][XU units]: a zero unit, input row oh + d(kh - 1)'s
//        W/8 units, a zero unit (XU odd).
// Rows outside the image and the zero units come from out-of-range offsets
// (the copy writes zeros).  Per 16-position step a lane reads its dout unit
// and, per kernel row, the x unit under its 8 positions and the neighbouring
// dwords; the horizontal shifts are v_alignbyte (dilation 1) or whole-dword
// selections (dilation 2).  Three LDS buffers, copies two stages ahead, one
// barrier a stage.  Partials are written as [split][tap][oc][ic].
template <int W, int DL>
struct WgGeo {
    static constexpr int KS = (W + 15) / 16;          // 16-position steps per row
    static constexpr int DU = (2 * KS) | 1;           // dout units per channel row
    static constexpr int XU = (W / 8 + 2) | 1;        // x units per (channel, kernel row)
    static constexpr int D_BYTES = 64 * DU * 16;
    // the x rows end in a zero unit, but the kw = 2 shift of a row's last
    // unit also reads the first dword after it: for the stage's last row
    // that is past the stage, so each stage ends in one more unit, zeroed
    // once and never copied over
    static constexpr int X_END = D_BYTES + 64 * 3 * XU * 16;
    static constexpr int STAGE = X_END + 16;
    static constexpr int INSTS = DU + 3 * XU;         // 1 KB copy instructions per stage
    static constexpr int PER_WAVE = (INSTS + 3) / 4;  // instructions of waves 0 .. INSTS % 4 - 1
};

template <int W, int DL>
__global__ __launch_bounds__(256, 1)
void wgrad3x3_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ dout, float *__restrict__ part,
                     int N, int C, int Co, int H, int rows_per) {
    using G = WgGeo<W, DL>;
    static_assert(3 * G::STAGE <= 160 * 1024, "three stages in LDS");
    __shared__ __align__(16) uint8_t smem[3 * G::STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int ic0 = blockIdx.x * 64, oc0 = blockIdx.y * 64, split = blockIdx.z;
    const int r32 = lane & 31, h = lane >> 5;
    const int NH = N * H;
    const int row_begin = split * rows_per;
    const int row_end = row_begin + rows_per < NH ? row_begin + rows_per : NH;
    const int plane_b = H * W * 2;                    // bytes per channel plane
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dout, (uint32_t)((int64_t)N * Co * H * W * 2));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)N * C * H * W * 2));

    // copy instructions of this wave: i = wave + 4 j; lane -> unit i * 64 + lane
    int n_mine = 0;
    uint32_t st_off[G::PER_WAVE];
    int st_kh[G::PER_WAVE];                           // -1: dout unit; 0..2: x kernel row; 3: zero unit
#pragma unroll
    for (int j = 0; j < G::PER_WAVE; ++j) {
        const int i = wave + 4 * j;
        st_off[j] = 0;
        st_kh[j] = 3;
        if (i >= G::INSTS) continue;
        ++n_mine;
        const int u = i * 64 + lane;
        if (i < G::DU) {
            const int oc = u / G::DU, uu = u - oc * G::DU;
            st_kh[j] = uu < W / 8 ? -1 : 3;
            st_off[j] = (uint32_t)(oc * plane_b + uu * 16);
        } else {
            const int ux = u - 64 * G::DU;
            const int ic = ux / (3 * G::XU), rem = ux - ic * (3 * G::XU);
            const int kh = rem / G::XU, uc = rem - kh * G::XU;
            st_kh[j] = (uc >= 1 && uc <= W / 8) ? kh : 3;
            st_off[j] = (uint32_t)(ic * plane_b + (uc - 1) * 16);
        }
    }
    auto issue = [&](int row, int buf) {
        const int n = row / H, oh = row - n * H;
        const uint32_t row_d = (uint32_t)(((n * Co + oc0) * H + oh) * W * 2);
        const uint32_t row_x = (uint32_t)(((n * C + ic0) * H + oh) * W * 2);
        lds_u8 *const base = (lds_u8 *)smem + buf * G::STAGE;
#pragma unroll
        for (int j = 0; j < G::PER_WAVE; ++j) {
            const int i = wave + 4 * j;
            if (i >= G::INSTS) break;
            const int kh = st_kh[j];
            if (i < G::DU) {
                dma_1k(base + i * 1024, dr, kh == -1 ? row_d + st_off[j] : kOob, 0);
            } else {
                const int ih = oh + DL * (kh - 1);
                const bool ok = kh < 3 && ih >= 0 && ih < H;
                dma_1k(base + i * 1024, xr, ok ? row_x + (uint32_t)(DL * (kh - 1) * W * 2) + st_off[j] : kOob, 0);
            }
        }
    };

    f32x16_t acc[9];
#pragma unroll
    for (int t = 0; t < 9; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;

    // operand offsets in a stage: A row wm*32 + r32 of dout, B row wn*32 + r32 of x
    const uint32_t a_off = (uint32_t)(((wm * 32 + r32) * G::DU + h) * 16);
    const uint32_t b_off = (uint32_t)(G::D_BYTES + ((wn * 32 + r32) * 3 * G::XU + 1 + h) * 16);
    auto compute = [&](int buf) {
        const uint8_t *sb = smem + buf * G::STAGE;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            const uint4 a = *reinterpret_cast<const uint4 *>(sb + a_off + ks * 32);
#pragma unroll
            for (int kh = 0; kh < 3; ++kh) {
                const uint8_t *xb = sb + b_off + (kh * G::XU + 2 * ks) * 16;
                const uint4 cur = *reinterpret_cast<const uint4 *>(xb);
                const uint32_t prv = *reinterpret_cast<const uint32_t *>(xb - 4);
                const uint32_t nxt = *reinterpret_cast<const uint32_t *>(xb + 16);
                const uint32_t c0 = cur.x, c1 = cur.y, c2 = cur.z, c3 = cur.w;
                // kw = 0: columns ow0-DL .. ow0+7-DL; kw = 1: the unit; kw = 2: ow0+DL .. ow0+7+DL
                uint4 b0, b2;
                if constexpr (DL == 1) {
                    b0 = make_uint4(__builtin_amdgcn_alignbyte(c0, prv, 2), __builtin_amdgcn_alignbyte(c1, c0, 2),
                                    __builtin_amdgcn_alignbyte(c2, c1, 2), __builtin_amdgcn_alignbyte(c3, c2, 2));
                    b2 = make_uint4(__builtin_amdgcn_alignbyte(c1, c0, 2), __builtin_amdgcn_alignbyte(c2, c1, 2),
                                    __builtin_amdgcn_alignbyte(c3, c2, 2), __builtin_amdgcn_alignbyte(nxt, c3, 2));
                } else {
                    // whole-dword shifts; fresh VALU results so the operand quads are built in registers
                    auto cp = [](uint32_t v) { return __builtin_amdgcn_perm(v, v, 0x03020100u); };
                    b0 = make_uint4(cp(prv), cp(c0), cp(c1), cp(c2));
                    b2 = make_uint4(cp(c1), cp(c2), cp(c3), cp(nxt));
                }
                acc[3 * kh + 0] = mfma32x32x16(a, b0, acc[3 * kh + 0]);
                acc[3 * kh + 1] = mfma32x32x16(a, cur, acc[3 * kh + 1]);
                acc[3 * kh + 2] = mfma32x32x16(a, b2, acc[3 * kh + 2]);
            }
        }
    };
    // wait until this wave's copies of all but the last `later` issued stages are done
    // (copies complete in order; the count is an immediate, so one branch per case)
    auto wait_all_but = [&](bool later) {
        if (!later) {
            CONV3X3_WAIT_VMCNT(0);
        } else if (n_mine == G::PER_WAVE) {
            CONV3X3_WAIT_VMCNT(G::PER_WAVE);
        } else {
            CONV3X3_WAIT_VMCNT(G::PER_WAVE - 1);
        }
    };

    if (tid < 3) *reinterpret_cast<uint4 *>(smem + tid * G::STAGE + G::X_END) = make_uint4(0, 0, 0, 0);
    const int rows = row_end > row_begin ? row_end - row_begin : 0;
    if (rows > 0) issue(row_begin, 0);
    if (rows > 1) issue(row_begin + 1, 1);
    wait_all_but(rows > 1);
    __syncthreads();
    for (int s = 0; s < rows; ++s) {
        const bool ahead = s + 2 < rows;
        if (ahead) issue(row_begin + s + 2, (s + 2) % 3);
        compute(s % 3);
        wait_all_but(ahead);                          // stage s + 1 copied
        __syncthreads();                              // stage s's buffer free, stage s + 1's visible
    }

    // part[split][tap][oc][ic]: 32 lanes on 32 consecutive input channels.
    // Through a buffer resource: the lane's part of the offset (its input
    // channel, the rows of its half) in one VGPR, the (tap, slot) part
    // uniform, so the 144 stores need no address registers of their own.
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(part + (int64_t)split * 9 * Co * C, (uint32_t)(9 * Co * C * 4));
    const int voff = ((oc0 + wm * 32 + 4 * h) * C + ic0 + wn * 32 + r32) * 4;
#pragma unroll
    for (int t = 0; t < 9; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[t][r]), pr, voff,
                                                  ((t * Co + 8 * (r >> 2) + (r & 3)) * C) * 4, 0);
}

// dw[oc][ic][tap] = sum over splits of part[split][tap][oc][ic], in a fixed
// order.  A workgroup takes 32 groups of 4 consecutive elements; thread
// (group, k) adds splits k*per .. k*per+per-1 in order with independent
// 16-byte loads (all in flight at once), then the 8 partial sums of a group
// are added in order k = 0 .. 7.  Each thread walking all splits by itself
// was latency-bound (17.5 us for 38 MB on the 3x3 layer).
__global__ __launch_bounds__(256)
void sum_splits_tap_kernel(const float *__restrict__ part, float *__restrict__ dw, int Co, int C, int splits) {
    __shared__ float4 red[8][32];
    const int g = threadIdx.x & 31, k = threadIdx.x >> 5;
    const int64_t n4 = (int64_t)9 * Co * C / 4;              // float4 groups (C % 64 == 0)
    const int64_t e4 = (int64_t)blockIdx.x * 32 + g;
    const int per = (splits + 7) / 8;
    const int i0 = k * per, i1 = i0 + per < splits ? i0 + per : splits;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e4 < n4) {
        const float4 *p = reinterpret_cast<const float4 *>(part) + e4;
#pragma unroll 8
        for (int i = i0; i < i1; ++i) {
            const float4 v = p[(int64_t)i * n4];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
    }
    red[k][g] = acc;
    __syncthreads();
    if (k != 0 || e4 >= n4) return;
    float4 sum = red[0][g];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        const float4 v = red[j][g];
        sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
    }
    const int64_t e = e4 * 4;                                  // (tap, oc, ic), ic fastest
    const int ic = (int)(e % C);
    const int64_t r = e / C;
    const int ocv = (int)(r % Co), tap = (int)(r / Co);
    float *d = dw + ((int64_t)ocv * C + ic) * 9 + tap;
    d[0] = sum.x; d[9] = sum.y; d[18] = sum.z; d[27] = sum.w;
}

bool wgrad3x3_ok(const Shape &sh) {
    return sh.ndim == 2 && sh.G == 1 && (sh.dil == 1 || sh.dil == 2) && sh.p == sh.dil && sh.K == 3 && sh.s == 1 &&
           sh.W % 8 == 0 && sh.W <= 64 && sh.C % 64 == 0 && (int64_t)9 * sh.Co * sh.C * 4 < (INT64_C(1) << 31) &&
           sh.Co % 64 == 0 && sh.x_elems() * 2 < (INT64_C(1) << 31) && sh.y_elems() * 2 < (INT64_C(1) << 31);
}

// dw[e] = sum over splits, in order, of part[split][e].
__global__ __launch_bounds__(256)
void sum_splits_kernel(const float *__restrict__ part, float *__restrict__ dw, int64_t n, int splits) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    float s = 0.f;
    for (int i = 0; i < splits; ++i) s += part[(int64_t)i * n + e];
    dw[e] = s;
}

// The same sum for n % 4 == 0 and 16-byte aligned part and dw, with the
// order of sum_splits_tap_kernel: thread (group g of 4 elements, k) adds
// splits k*per .. k*per+per-1 in order with independent 16-byte loads, then
// the 8 partial sums of a group are added in order k = 0 .. 7.
__global__ __launch_bounds__(256)
void sum_splits_vec_kernel(const float *__restrict__ part, float *__restrict__ dw, int64_t n4, int splits) {
    __shared__ float4 red[8][32];
    const int g = threadIdx.x & 31, k = threadIdx.x >> 5;
    const int64_t e4 = (int64_t)blockIdx.x * 32 + g;
    const int per = (splits + 7) / 8;
    const int i0 = k * per, i1 = i0 + per < splits ? i0 + per : splits;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e4 < n4) {
        const float4 *p = reinterpret_cast<const float4 *>(part) + e4;
#pragma unroll 8
        for (int i = i0; i < i1; ++i) {
            const float4 v = p[(int64_t)i * n4];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
    }
    red[k][g] = acc;
    __syncthreads();
    if (k != 0 || e4 >= n4) return;
    float4 sum = red[0][g];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        const float4 v = red[j][g];
        sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
    }
    reinterpret_cast<float4 *>(dw)[e4] = sum;
}

hipError_t launch_sum_splits(const float *part, float *out, int64_t n, int splits, hipStream_t st) {
    if (n % 4 == 0 && (uintptr_t)part % 16 == 0 && (uintptr_t)out % 16 == 0) {
        const int64_t n4 = n / 4;
        hipLaunchKernelGGL(sum_splits_vec_kernel, dim3((unsigned)((n4 + 31) / 32)), dim3(256), 0, st, part, out, n4,
                           splits);
    } else {
        hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, out, n, splits);
    }
    return hipGetLastError();
}

// Partial bias gradient: workgroup (oc, r) sums channel oc over images
// [r*per, min(N, (r+1)*per)), reading the images' rows of dout as one flat
// run of bf16 values (16 bytes a load when the base is 16-byte aligned and
// rows are whole 16-byte units);
// each thread adds its values in order, then a fixed-shape tree in LDS.
// part[r][oc] receives the sum, so the result does not depend on timing.
__global__ __launch_bounds__(256)
void bias_grad_part_kernel(const uint16_t *__restrict__ dout, float *__restrict__ part, int N, int Co,
                           int64_t plane, int per, int vec) {
    __shared__ float red[256];
    const int oc = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const int n0 = r * per, n1 = min(N, n0 + per);
    float s0 = 0.f, s1 = 0.f;
    if (vec) {
        const int64_t units = plane >> 3;                 // 16-byte units per image row
        const int64_t total = (int64_t)(n1 - n0) * units;
        for (int64_t u = tid; u < total; u += 256) {
            const int64_t n = n0 + u / units, q = u % units;
            const uint4 v = *(const uint4 *)(dout + ((n * Co + oc) * plane + q * 8));
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s0 += __uint_as_float(wv[j] << 16);
                s1 += __uint_as_float(wv[j] & 0xffff0000u);
            }
        }
    } else {
        const int64_t total = (int64_t)(n1 - n0) * plane;
        for (int64_t u = tid; u < total; u += 256) {
            const int64_t n = n0 + u / plane, q = u % plane;
            s0 += bf16_to_f32(dout[(n * Co + oc) * plane + q]);
        }
    }
    red[tid] = s0 + s1;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    if (tid == 0) part[(int64_t)r * Co + oc] = red[0];
}

}  // namespace

void launch_flip_weights_bf16(const Shape &sh, const uint16_t *w, uint16_t *wflip, hipStream_t st) {
    const int64_t total = sh.w_elems();
    hipLaunchKernelGGL(flip_weights_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, w, wflip,
                       sh.Cg(), sh.Cog(), sh.G, (int)sh.taps(), total);
}

int wgrad_splits(const Shape &sh, bool aligned) {
    if (aligned && wgrad3x3_ok(sh)) {
        // about 256 workgroups (one round of one per CU) over (C/64) x (C_out/64)
        // channel tiles, each a range of output rows: two rounds of shorter
        // ranges measured 8% slower on the 3x3 layer (twice the partials)
        const int64_t tiles = (int64_t)(sh.C / 64) * (sh.Co / 64);
        int64_t s = (256 + tiles - 1) / tiles;
        const int64_t rows = (int64_t)sh.N * sh.H;
        if (s > rows) s = rows;
        return (int)(s < 1 ? 1 : s);
    }
    if (wgrad_dw_ok(sh)) {
        // about 1024 workgroups: output channels x ranges of images
        int s = (1024 + sh.Co - 1) / sh.Co;
        return s < sh.N ? s : sh.N;
    }
    const int64_t P = sh.pixels();
    const int Kg = (int)sh.kgemm(), Cog = sh.Cog();
    const int bm = Cog > 64 ? 128 : 64;
    const int64_t tiles = (int64_t)((Kg + kBN - 1) / kBN) * ((Cog + bm - 1) / bm) * sh.G;
    int64_t s = (kTargetBlocks + tiles - 1) / tiles;
    const int64_t most = (P + 8 * kBK - 1) / (8 * kBK);        // at least 8 stages per range
    if (s > most) s = most;
    if (s < 1) s = 1;
    if (s > 256) s = 256;
    return (int)s;
}

int64_t wgrad_workspace_floats(const Shape &sh) {
    // the 3x3 kernel runs only on 16-byte aligned x and dout; size the
    // workspace for whichever route the pointers select
    // (and room for the bias partials after the weight ones)
    const int64_t per = sh.w_elems() + sh.Co;
    const int64_t a = (int64_t)wgrad_splits(sh, true) * per;
    const int64_t b = (int64_t)wgrad_splits(sh, false) * per;
    return a > b ? a : b;
}

hipError_t launch_wgrad_bf16(const Shape &sh, const uint16_t *x, const uint16_t *dout, float *part, float *dw,
                             float *db, hipStream_t st) {
    const int64_t P = sh.pixels();
    const int Kg = (int)sh.kgemm(), Cog = sh.Cog();
    // the bias gradient first, its partials in the front of the workspace
    // (the weight partials overwrite them afterwards, in stream order).  Folding
    // it into the 3x3 weight kernel measured slower (its channel-tile-0
    // workgroups, which set the makespan, took the extra LDS reads).
    // depthwise 3x3, stride 1, pad = dilation, W % 8 == 0: the weight kernel
    // also sums the bias gradient
    const bool dw3 = wgrad_dw_ok(sh) && sh.K == 3 && sh.s == 1 && (sh.dil == 1 || sh.dil == 2) && sh.p == sh.dil &&
                     sh.W % 8 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)dout % 16 == 0 &&
                     sh.x_elems() * 2 < (INT64_C(1) << 31) && sh.y_elems() * 2 < (INT64_C(1) << 31);
    // the general weight kernel (neither the 3x3 nor the depthwise one) also
    // sums the bias gradient from its dout tiles
    const bool aligned0 = (uintptr_t)x % 16 == 0 && (uintptr_t)dout % 16 == 0;
    const bool general = !(aligned0 && wgrad3x3_ok(sh)) && !wgrad_dw_ok(sh);
    if (db && !dw3 && !general) {
        const hipError_t e = launch_bias_grad_bf16(sh, dout, part, db, st);
        if (e != hipSuccess) return e;
    }
    const bool aligned = (uintptr_t)x % 16 == 0 && (uintptr_t)dout % 16 == 0;
    const int splits = wgrad_splits(sh, aligned);
    if (aligned && wgrad3x3_ok(sh)) {
        const int NH = sh.N * sh.H;
        const int per = (NH + splits - 1) / splits;
        const int used = (NH + per - 1) / per;             // ranges that hold rows
        dim3 grid((unsigned)(sh.C / 64), (unsigned)(sh.Co / 64), (unsigned)used);
#define WGRAD3X3_GO(WV)                                                                                           \
    if (sh.dil == 2)                                                                                              \
        hipLaunchKernelGGL((wgrad3x3_kernel<WV, 2>), grid, dim3(256), 0, st, x, dout, part, sh.N, sh.C, sh.Co, sh.H, \
                           per);                                                                                  \
    else                                                                                                          \
        hipLaunchKernelGGL((wgrad3x3_kernel<WV, 1>), grid, dim3(256), 0, st, x, dout, part, sh.N, sh.C, sh.Co, sh.H, \
                           per)
        switch (sh.W / 8) {
            case 1: WGRAD3X3_GO(8); break;
            case 2: WGRAD3X3_GO(16); break;
            case 3: WGRAD3X3_GO(24); break;
            case 4: WGRAD3X3_GO(32); break;
            case 5: WGRAD3X3_GO(40); break;
            case 6: WGRAD3X3_GO(48); break;
            case 7: WGRAD3X3_GO(56); break;
            default: WGRAD3X3_GO(64); break;
        }
#undef WGRAD3X3_GO
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t n4 = (int64_t)9 * sh.Co * sh.C / 4;
        hipLaunchKernelGGL(sum_splits_tap_kernel, dim3((unsigned)((n4 + 31) / 32)), dim3(256), 0, st, part, dw, sh.Co,
                           sh.C, used);
        return hipGetLastError();
    }
    if (wgrad_dw_ok(sh)) {
        const int per = (sh.N + splits - 1) / splits;
        const int used = (sh.N + per - 1) / per;          // ranges that hold images
        float *part_b = part + (int64_t)used * sh.w_elems();      // bias partials after the weight ones
        if (dw3 && sh.dil == 1)
            hipLaunchKernelGGL((wgrad_dw3_kernel<1>), dim3((unsigned)sh.Co, (unsigned)used), dim3(256), 0, st, sh, x,
                               dout, part, db ? part_b : nullptr, per);
        else if (dw3)
            hipLaunchKernelGGL((wgrad_dw3_kernel<2>), dim3((unsigned)sh.Co, (unsigned)used), dim3(256), 0, st, sh, x,
                               dout, part, db ? part_b : nullptr, per);
        else if (sh.K == 3)
            hipLaunchKernelGGL((wgrad_dw_kernel<3>), dim3((unsigned)sh.Co, (unsigned)used), dim3(256), 0, st, sh, x,
                               dout, part, used, per);
        else
            hipLaunchKernelGGL((wgrad_dw_kernel<0>), dim3((unsigned)sh.Co, (unsigned)used), dim3(256), 0, st, sh, x,
                               dout, part, used, per);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t n = sh.w_elems();
        const hipError_t e2 = launch_sum_splits(part, dw, n, used, st);
        if (e2 != hipSuccess) return e2;
        if (dw3 && db) return launch_sum_splits(part_b, db, (int64_t)sh.Co, used, st);
        return hipGetLastError();
    }
    const int64_t chunk = ((P + splits - 1) / splits + kBK - 1) / kBK * kBK;
    const int64_t plane = sh.out_plane();
    const int a_vec = (plane % 8 == 0) && ((uintptr_t)dout % 16 == 0);
    const bool b_vec = a_vec && sh.K == 1 && sh.Kd == 1 && sh.s == 1 && sh.sd == 1 && sh.p == 0 && sh.pd == 0 &&
                       ((uintptr_t)x % 16 == 0);
    const unsigned gx = (unsigned)((Kg + kBN - 1) / kBN);
    float *part_b = db ? part + (int64_t)splits * sh.w_elems() : nullptr;   // bias partials after the weight ones
    const int gmax = 65535 / splits;                    // groups per launch (grid z = splits * groups)
    for (int g0 = 0; g0 < sh.G; g0 += gmax) {
        const int ng = sh.G - g0 < gmax ? sh.G - g0 : gmax;
#define WGRAD_GO(BMV, BV)                                                                                    \
    hipLaunchKernelGGL((wgrad_kernel<BMV, BV>), dim3(gx, (unsigned)((Cog + BMV - 1) / BMV), (unsigned)(splits * ng)), \
                       dim3(256), 0, st, sh, x, dout, part, part_b, P, Kg, chunk, splits, g0, a_vec)
        if (Cog > 64) {
            if (b_vec) WGRAD_GO(128, 1); else WGRAD_GO(128, 0);
        } else {
            if (b_vec) WGRAD_GO(64, 1); else WGRAD_GO(64, 0);
        }
#undef WGRAD_GO
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t n = sh.w_elems();
    const hipError_t e3 = launch_sum_splits(part, dw, n, splits, st);
    if (e3 != hipSuccess || !db) return e3;
    return launch_sum_splits(part_b, db, (int64_t)sh.Co, splits, st);
}

int bias_grad_ranges(const Shape &sh) {
    // about 1024 workgroups, no more ranges than images, and the partials must
    // fit in the front of the weight-gradient workspace (which they use before
    // the weight kernels do)
    int64_t r = (1024 + sh.Co - 1) / sh.Co;
    if (r > sh.N) r = sh.N;
    const int64_t room = wgrad_workspace_floats(sh) / sh.Co;
    if (r > room) r = room;
    return (int)(r < 1 ? 1 : r);
}

hipError_t launch_bias_grad_bf16(const Shape &sh, const uint16_t *dout, float *part, float *db, hipStream_t st) {
    const int r = bias_grad_ranges(sh), per = (sh.N + r - 1) / r;
    const int ranges = (sh.N + per - 1) / per;
    hipLaunchKernelGGL(bias_grad_part_kernel, dim3((unsigned)sh.Co, (unsigned)ranges), dim3(256), 0, st, dout, part,
                       sh.N, sh.Co, sh.out_plane(), per,
                       (int)(sh.out_plane() % 8 == 0 && (uintptr_t)dout % 16 == 0));
    return launch_sum_splits(part, db, (int64_t)sh.Co, ranges, st);
}

}  // namespace convfwd
