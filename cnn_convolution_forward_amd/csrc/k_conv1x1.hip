// k_conv1x1.hip -- pointwise convolution (K = 1, stride 1, pad 0), bf16 in,
// fp32 accumulate and out, on the gfx950 matrix cores.
//
// With K = 1 the patch matrix X_col of "Why use matrix multiplication for
// convolution" (2.2) is the input itself: column (n, q) of X_col is the
// C_in-vector x[n, :, q], so Y_n = W_row @ X_n for every image, with W_row the
// (C_out, C_in) weight view (same page, 2.3) and X_n the (C_in, plane) slice
// of x.  No gather and no padding: the kernel is a plain GEMM whose B operand
// is read in NCHW order.
//
// Two kernels.  NCHW layers with C_in in {64, 128, 256} and C_out a
// multiple of 128 take the streaming kernel at the end of this file
// (persistent workgroups, weights held in registers, the stores of one tile
// overlapping the MFMAs of the next); the tiled kernel below takes the rest.
//
// Tiling: a workgroup computes 128 output channels x 128 output pixels (the
// pixel axis runs over N * plane, so a tile may straddle two images); four
// waves in a 2 x 2 grid, each 2 x 2 v_mfma_f32_32x32x16_bf16 tiles.  K loop in
// stages of 32 input channels, double-buffered in LDS and prefetched into
// registers one stage ahead.  Both operands land in LDS in memory order:
//   A  [oc 128][ic 32] (+8 pad) -- a 16-byte read gives a lane its 8 k;
//   B  [ic 32][px 128] (+16 pad) -- pixels contiguous as in NCHW; the
//      transposing LDS read ds_read_b64_tr_b16 turns four rows of 4-pixel
//      chunks into 4 consecutive k per pixel, two reads per fragment.
// Epilogue: + bias[oc]; fp32 stores go to y[n][oc][q], 32 lanes on 32
// consecutive pixels of one channel.
//
// The layer is bound by its output bytes (4 * C_out per pixel against 2 * C_in
// read), so the goal is a steady store stream: a small LDS footprint (38 KB)
// and at most 128 registers per lane let four workgroups share a CU (their
// loads and stores overlap each other's K loops), and block indices are mapped
// so that the C_out / 128 tiles of one pixel range run on the same XCD and
// read that pixel range from its L2 once.
//
// Requirements (checked by the launcher): K = 1, stride 1, pad 0, C_in % 32
// == 0, plane % 8 == 0, 16-byte aligned x and w, x, w and y below 2 GiB.
#include "conv_internal.h"
#include "conv3x3_common.h"

namespace convfwd {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kLdA = kBK + 8;     // 80-byte rows: 16-byte reads of 8 consecutive rows are conflict-free
constexpr int kLdB = kBN + 16;    // 288-byte rows: the 4 rows of a transposing read start 8 banks apart

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ uint2 read_tr(const uint16_t *p) {
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p));
    return __builtin_bit_cast(uint2, v);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
void conv1x1_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                    const float *__restrict__ bias, float *__restrict__ y,
                    int C, int Co, int plane, int64_t P, int npt, int ncb, int remap, int out_bf16, int relu,
                    int64_t xcs, int64_t xns) {
    __shared__ __align__(16) uint16_t As[2][kBM][kLdA];
    __shared__ __align__(16) uint16_t Bs[2][kBK][kLdB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // block -> (pixel tile, channel block); the ncb blocks of a pixel tile are
    // consecutive logical tiles, and each XCD (block % 8) runs a contiguous range.
    const int T = npt * ncb;
    int L = blockIdx.x;
    if (remap) L = (int)(blockIdx.x & 7) * (T >> 3) + (int)(blockIdx.x >> 3);
    const int pt = L / ncb, ob = L - pt * ncb;
    const int m0 = ob * kBM;
    const int64_t j0 = (int64_t)pt * kBN;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)(P / plane * C * plane * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)((int64_t)Co * C * 2));

    // loader units: A u -> (row u/4, k-quad u%4); B u -> (k row u/16, 8-pixel group u%16).
    // Element (k, image n, pixel q) of B is at x[k * xcs + n * xns + q]: NCHW
    // has xcs = plane, xns = C * plane.
    uint32_t a_off[2], b_off[2];
    const uint32_t b_step = (uint32_t)(kBK * xcs * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + 256 * i;
        const int row = u >> 2, kq = u & 3;
        a_off[i] = (m0 + row < Co) ? (uint32_t)(((int64_t)(m0 + row) * C + kq * 8) * 2) : kOob;
        const int kr = u >> 4, pu = u & 15;
        const int64_t px = j0 + pu * 8;
        if (px < P) {
            const int64_t n = px / plane, q = px - n * plane;
            b_off[i] = (uint32_t)((n * xns + kr * xcs + q) * 2);
        } else {
            b_off[i] = kOob;
        }
    }
    uint4 a_reg[2], b_reg[2];
    auto load = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            a_reg[i] = bload16(wr, a_off[i], (uint32_t)(kt * kBK * 2));
            b_reg[i] = bload16(xr, b_off[i], (uint32_t)kt * b_step);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = tid + 256 * i;
            *reinterpret_cast<uint4 *>(&As[buf][u >> 2][(u & 3) * 8]) = a_reg[i];
            *reinterpret_cast<uint4 *>(&Bs[buf][u >> 4][(u & 15) * 8]) = b_reg[i];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[i][0][r] = 0.f;
            acc[i][1][r] = 0.f;
        }

    // per-lane LDS coordinates of the operands
    const int a_row = wm * 64 + (lane & 31), a_k = 8 * (lane >> 5);
    const int b_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int b_col = wn * 64 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    const int nk = C / kBK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load(kt + 1);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            uint4 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const uint4 *>(&As[buf][a_row + i * 32][kk * 16 + a_k]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint2 lo = read_tr(&Bs[buf][kk * 16 + b_row][b_col + j * 32]);
                const uint2 hi = read_tr(&Bs[buf][kk * 16 + b_row + 4][b_col + j * 32]);
                b[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < nk) store(buf ^ 1);
        __syncthreads();
    }

    // epilogue: y[n][oc][q] = acc + bias[oc] (then ReLU, bf16 rounding), through
    // buffer resources (32-bit offsets; a bias resource with no records reads 0
    // when there is no bias).  Offsets are in fp32 elements * 4; a bf16 output
    // stores 2-byte elements at half those offsets.
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)(P * Co * (out_bf16 ? 2 : 4)));
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bias ? (const void *)bias : (const void *)y,
                                                bias ? (uint32_t)Co * 4 : 0u);
    uint32_t base[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t px = j0 + wn * 64 + j * 32 + (lane & 31);
        const int64_t n = px / plane, q = px - n * plane;
        base[j] = (px < P) ? (uint32_t)((n * Co * plane + q) * 4) : kOob;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int oc = m0 + wm * 64 + i * 32 + mfma32_row(r, lane);
            const float bv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(br, oc * 4, 0, 0));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bool ok = oc < Co && base[j] != kOob;
                const uint32_t vo = ok ? base[j] + (uint32_t)oc * plane * 4 : kOob;
                float v = acc[i][j][r] + bv;
                if (relu) v = fmaxf(v, 0.f);
                if (out_bf16)
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(v), yr, (int)(ok ? vo >> 1 : kOob),
                                                          0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yr, (int)vo, 0, 0);
            }
        }
}

// Channels-last pointwise layer: x is (pixels, C_in) and y (pixels, C_out),
// so Y = X @ W_row^T with both operands contiguous along the reduction (C_in):
// a tile of 128 pixels x 128 output channels, 32-channel stages, both
// operands staged in LDS as [row][k] and read in 16-byte pieces (no
// transposes).  The accumulator rows are pixels and its columns output
// channels, so 32 lanes store 32 consecutive channels of one pixel.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 4)))
void conv1x1_nhwc_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                         const float *__restrict__ bias, float *__restrict__ y,
                         int C, int Co, int64_t P, int npt, int ncb, int remap, int out_bf16, int relu) {
    constexpr int kLd = kBK + 8;          // 80-byte rows: 16-byte reads of 8 consecutive rows are conflict-free
    __shared__ __align__(16) uint16_t As[2][kBN][kLd];      // pixels x k
    __shared__ __align__(16) uint16_t Bs[2][kBM][kLd];      // output channels x k

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const int T = npt * ncb;
    int L = blockIdx.x;
    if (remap) L = (int)(blockIdx.x & 7) * (T >> 3) + (int)(blockIdx.x >> 3);
    const int pt = L / ncb, ob = L - pt * ncb;
    const int m0 = ob * kBM;                   // first output channel
    const int64_t j0 = (int64_t)pt * kBN;      // first pixel

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)(P * C * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)((int64_t)Co * C * 2));
    // loader units u -> (row u/4, k-quad u%4), two per thread for each operand
    uint32_t a_off[2], b_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + 256 * i;
        const int row = u >> 2, kq = u & 3;
        a_off[i] = (j0 + row < P) ? (uint32_t)(((j0 + row) * C + kq * 8) * 2) : kOob;
        b_off[i] = (m0 + row < Co) ? (uint32_t)(((int64_t)(m0 + row) * C + kq * 8) * 2) : kOob;
    }
    uint4 a_reg[2], b_reg[2];
    auto load = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            a_reg[i] = bload16(xr, a_off[i], (uint32_t)(kt * kBK * 2));
            b_reg[i] = bload16(wr, b_off[i], (uint32_t)(kt * kBK * 2));
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = tid + 256 * i;
            *reinterpret_cast<uint4 *>(&As[buf][u >> 2][(u & 3) * 8]) = a_reg[i];
            *reinterpret_cast<uint4 *>(&Bs[buf][u >> 2][(u & 3) * 8]) = b_reg[i];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[i][0][r] = 0.f;
            acc[i][1][r] = 0.f;
        }

    const int nk = C / kBK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load(kt + 1);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int kof = kk * 16 + (lane >> 5) * 8;
            uint4 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const uint4 *>(&As[buf][wm * 64 + i * 32 + (lane & 31)][kof]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const uint4 *>(&Bs[buf][wn * 64 + j * 32 + (lane & 31)][kof]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < nk) store(buf ^ 1);
        __syncthreads();
    }

    // y[pixel][oc] = acc + bias[oc] (then ReLU, bf16): lane column = output channel
    const int ob_ = out_bf16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)(P * Co * ob_));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int oc = m0 + wn * 64 + j * 32 + (lane & 31);
        const bool cok = oc < Co;
        const float bv = (bias && cok) ? bias[oc] : 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t px = j0 + wm * 64 + i * 32 + mfma32_row(r, lane);
                const bool ok = cok && px < P;
                const uint32_t vo = ok ? (uint32_t)((px * Co + oc) * ob_) : kOob;
                float v = acc[i][j][r] + bv;
                if (relu) v = fmaxf(v, 0.f);
                if (out_bf16)
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(v), yr, (int)vo, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yr, (int)vo, 0, 0);
            }
    }
}

// ---------------------------------------------------------------------------
// Streaming pointwise kernel: one persistent workgroup per CU, for NCHW with
// C_in in {64, 128, 256} and C_out a multiple of 128 (C_out / 128 dividing 32).
//
// The layer writes 2 * C_out / C_in times the bytes it reads, so the store
// stream has to run the whole time.  A workgroup owns one block of 128 output
// channels for the whole launch and walks a fixed list of 128-pixel tiles.
// Its eight waves form two groups of four (each group a 2 x 2 grid of 64 x 64
// MFMA blocks) that take the tiles in turn, in phases ended by the workgroup
// barrier: in phase p one group multiplies tile p while the other stores its
// tile p - 1 and copies the input of its next tile, p + 1, into its own LDS
// buffer -- so the MFMAs of one tile overlap the stores of the one before.
//   Weights: each wave holds its 64 channels x C_in of W_row in registers
//   (C_in / 2 registers per lane), read once from LDS after a coalesced copy.
//   Input tile: C_in rows x 128 pixels bf16 per group, copied straight into
//   LDS (32-byte segments of a row XORed with row % 4, so the four rows of a
//   transposing read land on distinct banks); one workgroup barrier a phase.
//   Counters: a storing wave issues the copy before its stores; the vector-
//   memory counter retires in issue order, so it waits for the copy with the
//   stores still in flight, and a multiplying wave issues no memory access.
// Workgroup g runs on XCD g % 8; the C_out / 128 channel blocks of a pixel
// tile sit on one XCD and walk its tiles together, so each XCD's L2 reads an
// input tile once.  Tile list of stream s: s, s + S, s + 2S, ... with S =
// 256 / (C_out / 128) streams.  LDS: 2 x C_in x 256 bytes + the bias block.
constexpr int kSWg = 256;                  // workgroups (one per CU)

template <int C, int OUTB, int RELU>
__global__ __launch_bounds__(512, 1)
void conv1x1_stream_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                           const float *__restrict__ bias, float *__restrict__ y,
                           int Co, int plane, int64_t P, int npt, int ncb) {
    constexpr int KS = C / 16;             // k-steps of one tile
    constexpr int DW = C / 16;             // 1 KB copies per wave per tile (C / 4 chunks of 4 rows, 4 waves)
    constexpr int TB = C * kBN * 2;        // bytes of one input tile
    __shared__ __align__(16) uint16_t Bs[2 * C * kBN];
    __shared__ __align__(16) float bsh[256];           // 128 bias values (+ the copy's zero-filled tail)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, gw = wave & 3;
    const int wm = gw >> 1, wn = gw & 1;

    const int g = blockIdx.x, xcd = g & 7, sl = g >> 3;
    const int ob = sl % ncb, stream = xcd + 8 * (sl / ncb);
    const int nstreams = kSWg / ncb;
    const int ntiles = stream < npt ? (npt - stream + nstreams - 1) / nstreams : 0;
    if (ntiles == 0) return;
    const int m0 = ob * kBM;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)(P * C * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)((int64_t)Co * C * 2));
    lds_u8 *const b_lds = (lds_u8 *)Bs;

    // bias: one 1 KB copy (lanes 32 .. 63 and a missing bias read zeros)
    if (wave == 0) {
        const __amdgpu_buffer_rsrc_t br = make_rsrc(bias ? (const void *)bias : (const void *)y, bias ? (uint32_t)Co * 4 : 0u);
        dma_1k((lds_u8 *)bsh, br, lane < 32 ? (uint32_t)(m0 * 4 + lane * 16) : kOob, 0);
    }

    // input copies: chunk c = rows 4c .. 4c+3; lane -> row 4c + lane / 16,
    // physical 16-byte unit lane % 16 holding logical unit l16 (pixels 8 l16 ..)
    const int r4 = lane >> 4, p16 = lane & 15;
    const int l16 = (((p16 >> 1) ^ r4) << 1) | (p16 & 1);
    // 32-bit offsets: x and y are below 2 GiB (checked by the launcher)
    const uint32_t uP = (uint32_t)P, uplane = (uint32_t)plane;
    auto b_voff = [&](int pt) -> uint32_t {
        const uint32_t px = (uint32_t)pt * kBN + 8 * l16;
        const uint32_t n = px / uplane, q = px - n * uplane;
        return px < uP ? ((n * C + r4) * uplane + q) * 2 : kOob;
    };
    auto copy_tile = [&](uint32_t vo) {
#pragma unroll
        for (int i = 0; i < DW; ++i) {
            const int ch = gw + 4 * i;
            dma_1k(b_lds + grp * TB + ch * 1024, xr, vo, ch * 4 * plane * 2);
        }
    };
    // prologue: the weight block goes through group 1's buffer (coalesced 1 KB
    // copies; [row 128][C/8 units], unit u of row r stored at u ^ (r % 8) so
    // that 16-byte reads of 8 consecutive rows are conflict-free) while group
    // 0's first tile lands in its own buffer
    constexpr int U = C / 8;
    for (int ch = wave; ch < 2 * U; ch += 8) {
        const int v = ch * 64 + lane, row = v / U, pu = v - row * U;
        dma_1k(b_lds + TB + ch * 1024, wr, (uint32_t)(((m0 + row) * C + (pu ^ (row & 7)) * 8) * 2), 0);
    }
    if (grp == 0) copy_tile(b_voff(stream));
    CONV3X3_WAIT_VMCNT(0);
    __syncthreads();
    // this wave's weights: fragment (kk, i) = row wm*64 + 32i + lane%32, unit
    // 2kk + lane/32, stored at (2kk + lane/32) ^ (lane % 8)
    uint4 areg[KS][2];
    {
        const int ta = (lane >> 5) ^ (lane & 7);
        const uint8_t *const Ab = reinterpret_cast<const uint8_t *>(Bs) + TB;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                areg[kk][i] = *reinterpret_cast<const uint4 *>(
                    Ab + ((wm * 64 + i * 32 + (lane & 31)) * U + ((2 * kk) ^ ta)) * 16);
    }
    __syncthreads();                // group 1's buffer is free again
    if (grp == 1 && ntiles > 1) copy_tile(b_voff(stream + nstreams));

    // B operand: rows 16kk + br and +4, 32-byte segment 4wn + (lane/16)%2 + 2j
    // stored at 4wn + (((lane/16)%2 + 2j) ^ rr), plus 8 bytes per lane % 4
    const int br = 8 * (lane >> 5) + ((lane & 15) >> 2), rr = (lane >> 2) & 3, g1 = (lane >> 4) & 1;
    uint32_t b_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        b_off[j] = (uint32_t)(grp * TB + br * kBN * 2 + (4 * wn + ((g1 + 2 * j) ^ rr)) * 32 + 8 * (lane & 3));
    const uint8_t *const Bb = reinterpret_cast<const uint8_t *>(Bs);

    constexpr int ob_ = OUTB ? 2 : 4;
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)(P * Co * ob_));
    const int ocl = wm * 64 + 4 * (lane >> 5);         // + 32i + 8(r/4) + r%4
    f32x16_t acc[2][2];

    for (int p = 0; p <= ntiles; ++p) {
        if (grp == (p & 1)) {
            if (p < ntiles) {          // multiply tile p
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        acc[i][0][r] = 0.f;
                        acc[i][1][r] = 0.f;
                    }
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    uint4 b[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const uint8_t *q = Bb + b_off[j] + kk * 16 * kBN * 2;
                        const uint2 lo = read_tr(reinterpret_cast<const uint16_t *>(q));
                        const uint2 hi = read_tr(reinterpret_cast<const uint16_t *>(q + 4 * kBN * 2));
                        b[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(areg[kk][i], b[j], acc[i][j]);
                }
            }
        } else if (p >= 1) {           // store tile p - 1, copy tile p + 1
            const int pt = stream + (p - 1) * nstreams;
            const bool more = p + 1 < ntiles;
            if (more) copy_tile(b_voff(stream + (p + 1) * nstreams));
            uint32_t base[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t px = (uint32_t)pt * kBN + wn * 64 + j * 32 + (lane & 31);
                const uint32_t n = px / uplane, q = px - n * uplane;
                base[j] = px < uP ? ((n * Co + m0 + ocl) * uplane + q) * ob_ : kOob;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int orow = i * 32 + 8 * (r >> 2) + (r & 3);
                    const float bv = bsh[ocl + orow];
                    const int soff = orow * plane * ob_;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        float v = acc[i][j][r] + bv;
                        if (RELU) v = fmaxf(v, 0.f);
                        if (OUTB)
                            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(v), yr, (int)base[j], soff, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yr, (int)base[j], soff, 0);
                    }
                }
            // the copy precedes the 64 stores: at most 63 outstanding means it has landed
            if (more) CONV3X3_WAIT_VMCNT(63);
        } else {                       // phase 0, group 1: its first tile, copied in the prologue
            CONV3X3_WAIT_VMCNT(0);
        }
        __syncthreads();
    }
}

}  // namespace

bool conv1x1_supported(const Shape &sh, const void *x, const void *w) {
    const int64_t plane = sh.out_plane();
    if (sh.nhwc)   // channels-last: any pixel count; x and y below 2 GiB
        return sh.plain() && sh.K == 1 && sh.s == 1 && sh.p == 0 && sh.C % kBK == 0 &&
               sh.x_elems() * 2 < (INT64_C(1) << 31) && sh.y_elems() * 4 < (INT64_C(1) << 31) &&
               sh.w_elems() * 2 < (INT64_C(1) << 31) && ((uintptr_t)x % 16) == 0 && ((uintptr_t)w % 16) == 0;
    return sh.plain() && sh.K == 1 && sh.s == 1 && sh.p == 0 && sh.C % kBK == 0 && plane % 8 == 0 &&
           plane < (INT64_C(1) << 31) && sh.x_elems() * 2 < (INT64_C(1) << 31) &&
           sh.y_elems() * 4 < (INT64_C(1) << 31) &&
           sh.w_elems() * 2 < (INT64_C(1) << 31) &&
           ((uintptr_t)x % 16) == 0 && ((uintptr_t)w % 16) == 0;
}

// The streaming kernel's shapes: NCHW, C_in in {64, 128, 256}, C_out / 128
// dividing 32 (one XCD's 32 workgroups hold whole groups of channel blocks).
static bool conv1x1_stream_ok(const Shape &sh) {
    const int ncb = sh.Co / kBM;
    return !sh.nhwc && (sh.C == 64 || sh.C == 128 || sh.C == 256) && sh.Co % kBM == 0 && ncb >= 1 && 32 % ncb == 0;
}

hipError_t launch_conv1x1_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w,
                               const float *bias, float *y, hipStream_t st) {
    const int64_t P = sh.pixels();
    const int plane = (int)sh.out_plane();
    const int npt = (int)((P + kBN - 1) / kBN);
    const int ncb = (sh.Co + kBM - 1) / kBM;
    if (conv1x1_stream_ok(sh)) {
#define CONV1X1_STREAM(CV)                                                                                        \
    if (sh.out_bf16) {                                                                                             \
        if (sh.relu) hipLaunchKernelGGL((conv1x1_stream_kernel<CV, 1, 1>), dim3(kSWg), dim3(512), 0, st, x, w, bias, y, sh.Co, plane, P, npt, ncb); \
        else hipLaunchKernelGGL((conv1x1_stream_kernel<CV, 1, 0>), dim3(kSWg), dim3(512), 0, st, x, w, bias, y, sh.Co, plane, P, npt, ncb);      \
    } else {                                                                                                       \
        if (sh.relu) hipLaunchKernelGGL((conv1x1_stream_kernel<CV, 0, 1>), dim3(kSWg), dim3(512), 0, st, x, w, bias, y, sh.Co, plane, P, npt, ncb); \
        else hipLaunchKernelGGL((conv1x1_stream_kernel<CV, 0, 0>), dim3(kSWg), dim3(512), 0, st, x, w, bias, y, sh.Co, plane, P, npt, ncb);      \
    }
        switch (sh.C) {
            case 64: CONV1X1_STREAM(64); break;
            case 128: CONV1X1_STREAM(128); break;
            default: CONV1X1_STREAM(256); break;
        }
#undef CONV1X1_STREAM
        return hipGetLastError();
    }
    const int64_t T = (int64_t)npt * ncb;
    const int remap = (T % 8 == 0) ? 1 : 0;
    if (sh.nhwc) {
        hipLaunchKernelGGL(conv1x1_nhwc_kernel, dim3((unsigned)T), dim3(256), 0, st, x, w, bias, y, sh.C, sh.Co, P, npt,
                           ncb, remap, sh.out_bf16, sh.relu);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(conv1x1_kernel, dim3((unsigned)T), dim3(256), 0, st, x, w, bias, y, sh.C, sh.Co,
                       plane, P, npt, ncb, remap, sh.out_bf16, sh.relu, (int64_t)plane, (int64_t)sh.C * plane);
    return hipGetLastError();
}

}  // namespace convfwd
