// k_conv3x3_cg.hip -- 3x3, stride 1, pad 1 convolution with column-group
// pixel fragments, bf16 in, fp32 accumulate and out, on the gfx950 matrix cores.
//
// The product is Y = W_row @ X_col ("Why use matrix multiplication for
// convolution", 2.3), with X_col never stored: for each chunk of 16 input
// channels the workgroup holds one halo tile of the input in LDS, and the nine
// taps of the kernel read it at shifted addresses ("Hand-writing Conv2D", 4.1:
// unfold a tile, multiply, discard).  Zero padding exists only in LDS.
//
// Pixel fragments.  A v_mfma_f32_32x32x16_bf16 operand covers 32 output
// pixels.  Here the 32 pixels of fragment c are 8 rows x 4 column groups:
// lane n holds row n % 8, column c + D * (n / 8), with D = W / 4.  Moving one
// column to the right maps fragment c onto fragment c + 1, so the horizontal
// taps (kw = 0, 1, 2) of fragments c .. c + J - 1 all read the same J + 2
// input fragments.  Kernel rows 1 and 2 read the same columns one and two
// input rows further down (a plain LDS read each: moving the row-0 fragment
// across lanes instead costs eight VALU operations per fragment between the
// MFMAs, which measured slower).  Per 16-channel stage a wave reads 9
// weight fragments and 3 (J + 2) input fragments for 9 J MFMAs (36 KB for
// 63 MFMAs at J = 7, against 126 KB when every tap reads both operands).
//
// Tiling: a workgroup computes 64 output channels x 8 output rows x W (one
// tile per workgroup), four waves in a 2 x 2 grid: 32 channels x J = D/2
// fragments each (J accumulator tiles, <= 128 accumulator registers).  Two
// workgroups share a CU (<= 256 registers per lane, <= 80 KB of LDS each), so
// one workgroup's prologue, barriers, epilogue and output drain overlap the
// other's MFMA work.  The K loop runs over 16-channel stages:
//   weights  [tap 9][oc 64][ic 16], 18 KB per stage, double-buffered, copied
//            by direct-to-LDS loads from the packed workspace
//            (launch_pack_w3x3, 128-channel blocks; a workgroup copies the
//            64-row half of each tap's block);
//   input    [row 10][col RP][ic 16] at 32 bytes per pixel, an odd row pitch
//            RP >= W + 2 and the two 16-byte halves swapped on bit 2 of the
//            row, so the 8 rows of a fragment column hit 8 distinct 16-byte
//            bank groups; double-buffered: stage s's input is loaded into
//            registers halfway through stage s - 2 and written transposed
//            (NCHW keeps channels strided, the operand needs 8 consecutive)
//            into the other buffer halfway through stage s - 1, so a whole
//            stage of MFMA work covers the load; one barrier a stage.
// Accumulator orientation D[px][oc]: lane l owns channel l % 32, and its 16
// slots are pixels (rows 4*(l/32) .. +3) x (4 column groups); across its J
// fragments a lane holds J consecutive columns of each (row, group).  The
// epilogue stages 32 channels at a time in LDS as [channel][row][column] and
// stores each channel's 8 rows (contiguous in y) in 8-byte pieces,
// consecutive lanes on consecutive pieces (bias is the accumulators' initial
// value).
//
// Dilation d (1 or 2, with pad d): a tile's 8 output rows are r0 + d*i, one
// row phase of a band of 8d rows, so kernel row kh of tile row i is again LDS
// row i + kh (the input rows are loaded d apart); a horizontal tap moves d
// fragment columns, so a pixel-wave steps through J + 2d input columns, and
// the LDS rows carry d halo columns on each side.
//
// Requirements (checked by the launcher): K = 3, s = 1, p = d, groups 1, C_in % 16 == 0,
// C_out % 128 == 0, W % 8 == 0, 32 <= W <= 64, packed weights, 16-byte
// aligned x.
#include <stdlib.h>

#include "conv_internal.h"
#include "conv3x3_common.h"

namespace convfwd {
namespace {

constexpr int kThreads = 256;
constexpr int kOc = 64;                  // output channels per workgroup
constexpr int kPackOcBlock = 128;        // channel block of the packed weight layout
constexpr int kIc = 16;                  // input channels per stage
constexpr int kRows = 8;                 // output rows per tile
constexpr int kInRows = kRows + 2;       // input rows per tile (halo)
constexpr int kPix = 32;                 // LDS bytes per input pixel: 16 bf16, halves swizzled by row
constexpr int kTapBytes = kOc * 32;      // one tap's weights in LDS (2 KB)
constexpr int kWStage = 9 * kTapBytes;   // 18432 bytes of weights per stage
constexpr int kPackStage = 9 * kPackOcBlock * 32;   // 36864: one stage of a packed 128-channel block
constexpr int kEpiOc = 32;               // channels per epilogue pass

// 16-byte half of an input pixel that holds channels 8h .. 8h+7 in LDS
// input row rho: the halves swap on bit 2 of the row, so the 8 rows of a
// fragment column (32-byte pixels, odd row pitch) hit 8 distinct 16-byte
// bank groups.
__device__ __forceinline__ int in_half(int h, int rho) { return h ^ ((rho >> 2) & 1); }

template <int D, int DL>
struct Geo {
    static constexpr int W = 4 * D;
    static constexpr int J = D / 2;                       // fragments per pixel-wave
    static constexpr int Q = J + 2 * DL;                  // input fragment columns per pixel-wave
    static constexpr int RP = (W + 2 * DL) | 1;           // odd input row pitch (pixels), DL halo columns each side
    static constexpr int IN_BYTES = kInRows * RP * kPix;
    static constexpr int LDS = 2 * kWStage + 2 * IN_BYTES;
    static constexpr int UNITS = 2 * kInRows * (W / 8);   // input load units per stage
};

// Zero the halo columns (the DL left and RP - W - DL right ones, 32 bytes per
// pixel) of nb consecutive input images [row 10][col RP] at dst.
template <int W, int RP, int DL>
__device__ __forceinline__ void zero_halo(uint8_t *dst, int nb, int tid) {
    constexpr int HC = RP - W;
    for (int i = tid; i < nb * kInRows * HC * 2; i += kThreads) {
        const int hh = i & 1, rest = i >> 1;
        const int c = rest % HC, rb = rest / HC;            // rb = image * 10 + row
        const int col = c < DL ? c : W + c;
        reinterpret_cast<uint4 *>(dst + (rb * RP + col) * kPix)[hh] = make_uint4(0, 0, 0, 0);
    }
}

template <bool V>
struct BoolC {
    static constexpr bool value = V;
};
template <int V>
struct IntC {
    static constexpr int value = V;
};

// The MFMAs of input-fragment column q (column c0 - 1 + q of this wave's
// range) and kernel row rr: the fragment serves output fragment j = q - kw
// for the three horizontal taps kw.
template <int D, int DL, int RR>
__device__ __forceinline__ void cg_mfma(f32x16_t (&acc)[(Geo<D, DL>::J)], const uint4 (&A)[9], const uint4 &b, int q) {
    constexpr int J = Geo<D, DL>::J;
#pragma unroll
    for (int kw = 0; kw < 3; ++kw) {
        const int j = q - DL * kw;
        if (j >= 0 && j < J) acc[j] = mfma32x32x16(b, A[RR * 3 + kw], acc[j]);
    }
}

// Column step q.  The fragments of kernel rows 0, 1 and 2 of column q are
// three LDS reads, one input row apart (ib, tb, ub).  A step first issues
// the reads of column q + 1, then the 9 (or fewer) MFMAs of column q, so the
// reads have a column of MFMA work to arrive.  A scheduling barrier keeps the
// compiler from sinking those reads between the column's MFMAs, where they
// had only one or two MFMAs to arrive (0.8% faster on the 3x3 layer, five
// alternating rounds on one box).
template <int D, int DL, int q, class Mid>
__device__ __forceinline__ void cg_col(f32x16_t (&acc)[(Geo<D, DL>::J)], const uint4 (&A)[9], uint4 (&B0)[2],
                                       uint4 (&T1)[2], uint4 (&T2)[2], const uint8_t *ib, const uint8_t *tb,
                                       const uint8_t *ub, Mid &&mid) {
    constexpr int Q = Geo<D, DL>::Q;
    if constexpr (q + 1 < Q) {
        B0[(q + 1) & 1] = *reinterpret_cast<const uint4 *>(ib + (q + 1) * kPix);
        T1[(q + 1) & 1] = *reinterpret_cast<const uint4 *>(tb + (q + 1) * kPix);
        T2[(q + 1) & 1] = *reinterpret_cast<const uint4 *>(ub + (q + 1) * kPix);
        __builtin_amdgcn_sched_barrier(0);
    }
    cg_mfma<D, DL, 0>(acc, A, B0[q & 1], q);
    cg_mfma<D, DL, 1>(acc, A, T1[q & 1], q);
    cg_mfma<D, DL, 2>(acc, A, T2[q & 1], q);
    // the middle-of-stage work in five parts over the columns from Q/2 - 1
    // (the last ones share the final column when Q is small): the input
    // fragments' transposing writes in two halves, the next weights' copies,
    // the input loads in two halves.  In one piece at column Q/2 the stage
    // took 0.5-1% longer (five alternating rounds on one box).
    if constexpr (q == (Q / 2 - 1 < Q - 1 ? Q / 2 - 1 : Q - 1)) mid(IntC<0>{});
    if constexpr (q == (Q / 2 < Q - 1 ? Q / 2 : Q - 1)) mid(IntC<1>{});
    if constexpr (q == (Q / 2 + 1 < Q - 1 ? Q / 2 + 1 : Q - 1)) mid(IntC<2>{});
    if constexpr (q == (Q / 2 + 2 < Q - 1 ? Q / 2 + 2 : Q - 1)) mid(IntC<3>{});
    if constexpr (q == (Q / 2 + 3 < Q - 1 ? Q / 2 + 3 : Q - 1)) mid(IntC<4>{});
    if constexpr (q + 1 < Q) cg_col<D, DL, q + 1>(acc, A, B0, T1, T2, ib, tb, ub, mid);
}

// Epilogue of a column-group tile (64 output channels x 8 output rows r0 +
// DL*i x W of image n, channels ocb ..).  Two passes of 32 channels through
// LDS: in pass p wave row p writes its accumulators into the pass image
// [channel 32][row 8][column W] (fp32, channel pitch 8W + 2 dwords), then all
// four waves read it back and store it.
//   Writes: a lane holds J consecutive columns c0 .. c0+J-1 of each (row,
//   column group); they go out as 4-byte writes at immediate offsets from one
//   lane base (paired by the compiler).  The pitch 8W + 2 puts 32 channels on
//   16 banks: a 2-way conflict, against 4-way with half the lanes idle for a
//   pitch of 8W + 4 and 16 channels a pass.  (An odd pitch would make the
//   writes conflict-free but misalign the 8-byte readback; 8-byte writes need
//   register pairs the accumulator layout does not give.)
//   Readback (NCHW): a wave reads one channel at a time, lane i on the 8-byte
//   units i, i+64, ... of that channel's 8 rows (consecutive in LDS), and
//   stores each unit's 2 fp32 (or 4 bf16) outputs with one 8-byte store: the
//   lane's output offsets are fixed for the whole epilogue and the channel
//   comes in as the scalar offset, so no address is computed per chunk.
//   Readback (NHWC): 16-byte chunks of one pixel's channels.
template <int W>
struct EpiGeo {
    static constexpr int P = kRows * W + 2;        // channel pitch (dwords), 2 x odd
    // a lane's last readback unit may lie past the last channel's 8 rows
    // (units are read in steps of 64): 64 units of 8 (fp32 out) or 16 (bf16
    // out) bytes per step
    static constexpr int T2 = 64 * ((4 * W + 63) / 64) * 8, T4 = 64 * ((2 * W + 63) / 64) * 16;
    static constexpr int TAIL = P * 4 > (T2 > T4 ? T2 : T4) ? P * 4 : (T2 > T4 ? T2 : T4);
    static constexpr int BYTES = (kEpiOc - 1) * P * 4 + TAIL;
};


template <int D, int OUT, int NHWC, int DL>
__device__ __forceinline__ void cg_epilogue(uint8_t *smem, const f32x16_t (&acc)[(Geo<D, DL>::J)], float *y, int n,
                                            int Co, int ocb, int H, int r0, int relu) {
    using G = Geo<D, DL>;
    constexpr int W = G::W, J = G::J;
    constexpr int P = EpiGeo<W>::P;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int c0 = wn * J;
    const int HW = H * W;
    float *const epi = reinterpret_cast<float *>(smem);
    constexpr int kOutB = OUT ? 2 : 4;                   // bytes per output element
    // NCHW: this tile's 64 channel planes; NHWC: the image (pixel-major, C_out channels each)
    const __amdgpu_buffer_rsrc_t yr =
        NHWC ? make_rsrc((char *)y + (int64_t)n * HW * Co * kOutB, (uint32_t)HW * Co * kOutB)
             : make_rsrc((char *)y + ((int64_t)n * Co + ocb) * HW * kOutB, (uint32_t)kOc * HW * kOutB);
    // writer lane: channel l32 of the pass, rows 4h .. 4h+3; slot r of
    // fragment j is (row 4h + r%4, column c0 + j + D*(r/4))
    float *const wdst = epi + l32 * P + 4 * h * W + c0;

    // NCHW readback: 8-byte units of fp32 (2 values, or 4 for bf16 output),
    // kU per channel, lane on units lane + 64*it
    constexpr int kF = OUT ? 4 : 2;                      // fp32 values read per store
    constexpr int kU = kRows * W / kF;
    constexpr int kIt = (kU + 63) / 64;
    uint32_t voff[kIt];
    if (!NHWC) {
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int u = lane + 64 * it, e = u * kF;
            const int row = e / W, col = e - row * W, orow = r0 + DL * row;
            voff[it] = (u < kU && orow < H) ? (uint32_t)((orow * W + col) * kOutB) : kOob;
        }
    }

#pragma unroll
    for (int p = 0; p < 2; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        if (wm == p) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float *base = wdst + (r & 3) * W + (r >> 2) * D;
#pragma unroll
                for (int j = 0; j < J; ++j) base[j] = acc[j][r];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        // the ReLU choice is one uniform branch around the whole readback
        auto readback = [&](auto rc) {
            constexpr bool R = decltype(rc)::value;
            if (NHWC) {
                // chunk = (pixel, group of kPer channels of this pass)
                constexpr int kPer = 16 / kOutB;
                constexpr int kq = kEpiOc / kPer;
                constexpr int kChunks = kRows * W * kq;
    #pragma unroll
                for (int k = 0; k < (kChunks + kThreads - 1) / kThreads; ++k) {
                    const int cid = k * kThreads + tid;
                    if (kChunks % kThreads == 0 || cid < kChunks) {
                        const int px = cid / kq, qd = cid - px * kq;
                        const int row = px / W, col = px - row * W;
                        const int orow = r0 + DL * row;
                        const uint32_t vo =
                            orow < H ? (uint32_t)(((orow * W + col) * Co + ocb + p * kEpiOc + qd * kPer) * kOutB) : kOob;
                        float f[8];
    #pragma unroll
                        for (int u = 0; u < kPer; ++u) f[u] = epi[(qd * kPer + u) * P + row * W + col];
                        u32x4_t va;
                        if (OUT == 0) {
    #pragma unroll
                            for (int u = 0; u < 4; ++u) va[u] = __float_as_uint(R ? fmaxf(f[u], 0.f) : f[u]);
                        } else {
                            uint32_t b[8];
    #pragma unroll
                            for (int u = 0; u < 8; ++u) b[u] = f32_to_bf16_rne(R ? fmaxf(f[u], 0.f) : f[u]);
                            va = (u32x4_t){b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16),
                                           b[6] | (b[7] << 16)};
                        }
                        __builtin_amdgcn_raw_buffer_store_b128(va, yr, (int)vo, 0, 0);
                    }
                }
            } else {
                // wave w: channels 8w .. 8w+7 of the pass
    #pragma unroll
                for (int i = 0; i < kEpiOc / 4; ++i) {
                    const int c = wave * (kEpiOc / 4) + i;
                    const float *src = epi + c * P + lane * kF;
                    const uint32_t soff = (uint32_t)((p * kEpiOc + c) * HW * kOutB);
    #pragma unroll
                    for (int it = 0; it < kIt; ++it) {
                        float f[4];
                        const float2 a = *reinterpret_cast<const float2 *>(src + it * 64 * kF);
                        f[0] = a.x; f[1] = a.y;
                        if (OUT) {
                            const float2 b = *reinterpret_cast<const float2 *>(src + it * 64 * kF + 2);
                            f[2] = b.x; f[3] = b.y;
                        }
                        u32x2_t va;
                        if (OUT == 0) {
                            va[0] = __float_as_uint(R ? fmaxf(f[0], 0.f) : f[0]);
                            va[1] = __float_as_uint(R ? fmaxf(f[1], 0.f) : f[1]);
                        } else {
                            uint32_t b[4];
    #pragma unroll
                            for (int u = 0; u < 4; ++u) b[u] = f32_to_bf16_rne(R ? fmaxf(f[u], 0.f) : f[u]);
                            va[0] = b[0] | (b[1] << 16);
                            va[1] = b[2] | (b[3] << 16);
                        }
                        __builtin_amdgcn_raw_buffer_store_b64(va, yr, (int)voff[it], (int)soff, 0);
                    }
                }
            }
        };
        if (relu) readback(BoolC<true>{}); else readback(BoolC<false>{});
        if (p < 1) __syncthreads();
    }
}

// OUT: 0 = fp32 output, 1 = bf16 output (rounded to nearest even); relu:
// max(y, 0) before the store.  NHWC: x and y channels-last -- the loader
// then copies each pixel's 8 channels as they are (no transpose) and the
// epilogue writes each pixel's channels contiguously.
template <int D, int OUT, int NHWC, int DL>
__global__ __launch_bounds__(kThreads, 2)
void conv3x3cg_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wp,
                      const float *__restrict__ bias, float *__restrict__ y,
                      int C, int H, int Co, int rb_per_img, int remap, int relu) {
    using G = Geo<D, DL>;
    constexpr int W = G::W, J = G::J, RP = G::RP;
    __shared__ __align__(16) uint8_t smem[G::LDS];
    static_assert(G::LDS >= EpiGeo<W>::BYTES, "the epilogue image overlays the stage buffers");
    static_assert(G::LDS <= 80 * 1024, "two workgroups per CU");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    // block -> (tile, channel half); the two halves of a tile are neighbours,
    // and with remap consecutive tiles (which share halo rows) run on one XCD
    // (block b runs on XCD b % 8)
    const int T = gridDim.x;
    int t = blockIdx.x;
    if (remap) t = (int)(blockIdx.x & 7) * (T >> 3) + (int)(blockIdx.x >> 3);
    const int half = t & 1;
    t >>= 1;
    // image n; within it, band tr / DL of 8 * DL rows and its row phase tr % DL:
    // output rows r0 + DL * i for i = 0 .. 7
    const int n = t / rb_per_img;
    const int tr = t - n * rb_per_img, band = tr / DL;
    const int r0 = band * kRows * DL + (tr - band * DL);
    const int ocb = (int)blockIdx.y * kPackOcBlock + half * kOc;
    const int HW = H * W;
    const int S = C / kIc;

    uint8_t *const wbuf = smem;
    uint8_t *const ibuf = smem + 2 * kWStage;
    lds_u8 *const wlds = (lds_u8 *)smem;

    // ---- input loader: unit u -> (row rho, 8-pixel group pg, channel half g8);
    // rows fastest so neighbouring lanes write LDS rows RP pixels apart
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (int64_t)n * C * HW, (uint32_t)C * HW * 2);
    const bool in_active = tid < G::UNITS;
    const bool x_wave = wave * 64 < G::UNITS;   // this wave has lanes that own units (and issues their loads)
    const int rho = tid % kInRows, rest = tid / kInRows;
    const int pg = rest % (W / 8), g8 = in_active ? rest / (W / 8) : 0;
    const int ih = r0 - DL + DL * rho;        // LDS row rho holds input row r0 - DL + DL * rho
    const bool ivalid = in_active && ih >= 0 && ih < H;
    // NCHW: channel g8*8 + e's 8 pixels are 16 contiguous bytes (e = channel);
    // NHWC: pixel pg*8 + e's channels g8*8 .. +7 are (e = pixel)
    const uint32_t ivoff = !ivalid ? kOob
                           : NHWC ? (uint32_t)(((ih * W + pg * 8) * C + g8 * 8) * 2)
                                  : (uint32_t)((g8 * 8 * HW + ih * W + pg * 8) * 2);
    const uint32_t idst = (uint32_t)((rho * RP + pg * 8 + DL) * kPix + in_half(g8, rho) * 16);
    const uint32_t chan_bytes = (uint32_t)HW * 2, stage_bytes = NHWC ? (uint32_t)kIc * 2 : chan_bytes * kIc;
    const uint32_t e_bytes = NHWC ? (uint32_t)C * 2 : chan_bytes;
    uint4 xin[8];
    // only the lanes that own a unit load (a wave with none issues nothing:
    // the loads of idle lanes would still occupy the address units)
    auto load_x = [&](int s, int e0 = 0, int e1 = 8) {
        if (!in_active) return;
#pragma unroll
        for (int e = e0; e < e1; ++e) xin[e] = bload16(xr, ivoff + e * e_bytes, (uint32_t)s * stage_bytes);
    };
    auto store_x = [&](int buf, int j0 = 0, int j1 = 8) {
        if (!in_active) return;
        if (NHWC) {
            uint8_t *dst = ibuf + buf * G::IN_BYTES + idst;
#pragma unroll
            for (int j = j0; j < j1; ++j) *reinterpret_cast<uint4 *>(dst + j * kPix) = xin[j];
            return;
        }
        const uint32_t *v = reinterpret_cast<const uint32_t *>(xin);   // v[e*4 + j/2]: channel e, pixels j, j+1
        uint8_t *dst = ibuf + buf * G::IN_BYTES + idst;
#pragma unroll
        for (int j = j0; j < j1; ++j) {
            const int dj = j >> 1, hj = j & 1;
            uint4 o;
            o.x = pack_halves(v[0 * 4 + dj], hj, v[1 * 4 + dj], hj);
            o.y = pack_halves(v[2 * 4 + dj], hj, v[3 * 4 + dj], hj);
            o.z = pack_halves(v[4 * 4 + dj], hj, v[5 * 4 + dj], hj);
            o.w = pack_halves(v[6 * 4 + dj], hj, v[7 * 4 + dj], hj);
            *reinterpret_cast<uint4 *>(dst + j * kPix) = o;
        }
    };
    // ---- weights: 18 x 1 KB blocks per stage (tap t, sub-block u: rows
    // 32u .. 32u+31 of this workgroup's 64-row half of the packed block);
    // wave w copies blocks w, w + 4, ...
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp + (int64_t)blockIdx.y * kPackOcBlock * C * 9,
                                                (uint32_t)kPackOcBlock * C * 9 * 2);
    const uint32_t lane16 = (uint32_t)lane * 16;
    auto dma_w = [&](int s, int buf) {
        for (int blk = wave; blk < 18; blk += 4) {
            const int tap = blk >> 1, u = blk & 1;
            dma_1k(wlds + buf * kWStage + tap * kTapBytes + u * 1024, wr, lane16,
                   s * kPackStage + tap * (kPackOcBlock * 32) + half * kTapBytes + u * 1024);
        }
    };

    // operand addresses: A (weights) row wm*32 + l32 of the tap, k half h
    // (swizzled on the row's bits 2-3, which the 64-row offset leaves alone);
    // B (input fragment) for fragment column c' = c0 - 1 + q at kernel row rr
    // is at (input row (l32 % 8) + rr, column c' + D*(l32 / 8)), with the
    // 16-byte half swizzled on that input row: b_base, b1_base, b2_base for
    // rr = 0, 1, 2, plus q * 32
    const uint32_t a_off = (uint32_t)((wm * 32 + l32) * 32 + ((h ^ wswz(l32)) * 16));
    const int c0 = wn * J;
    const uint32_t b_base = (uint32_t)((((l32 & 7) * RP) + D * (l32 >> 3) + c0) * kPix +
                                       in_half(h, l32 & 7) * 16);
    const uint32_t b1_base = (uint32_t)(((((l32 & 7) + 1) * RP) + D * (l32 >> 3) + c0) * kPix +
                                        in_half(h, (l32 & 7) + 1) * 16);
    const uint32_t b2_base = (uint32_t)(((((l32 & 7) + 2) * RP) + D * (l32 >> 3) + c0) * kPix +
                                        in_half(h, (l32 & 7) + 2) * 16);

    // zero the halo columns of both input buffers (DL on the left, RP - W -
    // DL on the right): the loader writes every other column of all 10 rows
    // each stage (rows outside the image as zeros) and never these
    zero_halo<W, RP, DL>(ibuf, 2, tid);

    // ---- prologue: stage 0
    dma_w(0, 0);
    load_x(0);
    const float bv = bias ? bias[ocb + wm * 32 + l32] : 0.f;
    CONV3X3_WAIT_VMCNT(0);
    store_x(0);
    if (S > 1) load_x(1);            // stored at the middle of stage 0
    __syncthreads();

    // accumulators start at this lane's channel bias
    f32x16_t acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = bv;

    for (int s = 0; s < S; ++s) {
        const int b = s & 1;
        const bool more = s + 1 < S;
        const uint8_t *wb = wbuf + b * kWStage + a_off;
        const uint8_t *ib = ibuf + b * G::IN_BYTES + b_base;
        const uint8_t *tb = ibuf + b * G::IN_BYTES + b1_base;
        const uint8_t *ub = ibuf + b * G::IN_BYTES + b2_base;
        uint4 A[9], B0[2], T1[2], T2[2];
#pragma unroll
        for (int t = 0; t < 9; ++t) A[t] = *reinterpret_cast<const uint4 *>(wb + t * kTapBytes);
        B0[0] = *reinterpret_cast<const uint4 *>(ib);
        T1[0] = *reinterpret_cast<const uint4 *>(tb);
        T2[0] = *reinterpret_cast<const uint4 *>(ub);
        // halfway through the stage the next stage's input (loaded halfway
        // through the previous stage, so a whole stage of MFMA work covers
        // its latency) goes into the other buffers, which nobody reads this
        // stage; then the next stage's weights are copied and the input of
        // the stage after is loaded.  The weight copies are issued after
        // the wait for the input (and before the next input loads) because
        // the compiler does not count them: its own wait before the input
        // is used only has to cover the input loads, and loads complete in
        // issue order, so the copies are waited for separately at the end
        // of the stage, with the next input still in flight.
        auto mid = [&](auto ph) {
            constexpr int P = decltype(ph)::value;
            if (more) {
                if constexpr (P == 0) {
                    CONV3X3_WAIT_VMCNT(0);
                    store_x(b ^ 1, 0, 4);
                }
                if constexpr (P == 1) store_x(b ^ 1, 4, 8);
                if constexpr (P == 2) dma_w(s + 1, b ^ 1);
                if constexpr (P == 3) {
                    if (s + 2 < S) load_x(s + 2, 0, 4);
                }
                if constexpr (P == 4) {
                    if (s + 2 < S) load_x(s + 2, 4, 8);
                }
            }
        };
        // raised priority over the MFMA columns: while this wave is between
        // stages (loads, transposes, the barrier) the CU's other workgroup
        // issues, and while both multiply the arbiter favours MFMA issue
        // (1.8% faster on the 3x3 layer than without)
        __builtin_amdgcn_s_setprio(1);
        cg_col<D, DL, 0>(acc, A, B0, T1, T2, ib, tb, ub, mid);
        __builtin_amdgcn_s_setprio(0);
        // the next stage's weights have landed (the input loads issued
        // after them, 8 by each wave that owns input units, may still be in
        // flight; a wave without units issued none, so it waits for all)
        if (more) {
            if (s + 2 < S && x_wave) CONV3X3_WAIT_VMCNT(8);
            else CONV3X3_WAIT_VMCNT(0);
        }
        __syncthreads();            // this stage's buffers free, the next stage's visible
    }

    cg_epilogue<D, OUT, NHWC, DL>(smem, acc, y, n, Co, ocb, H, r0, relu);
}

// Grouped layers with 32 output channels per group (C_in/G a multiple of
// 16): a workgroup's 64 output channels are two whole groups, and wave row
// wm works on group gA + wm with an input plane of its own (the same pixel
// layout as above, one plane per group).  Weights are packed as for a layer
// of C_in/G input channels, so stage s of an output channel holds its own
// group's channels 16s .. 16s+15.  Both planes and the weights of a stage are
// single-buffered (56 KB at W = 56): load, barrier, MFMAs, barrier.  Groups
// of 32 channels make short K loops (C_in/G / 16 stages), so the other
// workgroup on the CU, not a pipeline inside this one, covers the loads.
template <int D, int OUT>
__global__ __launch_bounds__(kThreads, 2)
void conv3x3cg_gp_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wp,
                         const float *__restrict__ bias, float *__restrict__ y,
                         int C, int H, int Co, int Cg, int rb_per_img, int remap, int relu) {
    using G = Geo<D, 1>;
    constexpr int W = G::W, J = G::J, RP = G::RP;
    constexpr int kLds = kWStage + 2 * G::IN_BYTES;
    constexpr int kEpiB = EpiGeo<W>::BYTES;
    __shared__ __align__(16) uint8_t smem[kLds > kEpiB ? kLds : kEpiB];
    static_assert(kLds <= 80 * 1024, "two workgroups per CU");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const int T = gridDim.x;
    int t = blockIdx.x;
    if (remap) t = (int)(blockIdx.x & 7) * (T >> 3) + (int)(blockIdx.x >> 3);
    const int half = t & 1;
    t >>= 1;
    const int n = t / rb_per_img;
    const int r0 = (t - n * rb_per_img) * kRows;
    const int ocb = (int)blockIdx.y * kPackOcBlock + half * kOc;
    const int gA = ocb / 32;                  // group of wave row 0; wave row 1 takes gA + 1
    const int HW = H * W;
    const int S = Cg / kIc;

    uint8_t *const wbuf = smem;
    uint8_t *const ibuf = smem + kWStage;
    lds_u8 *const wlds = (lds_u8 *)smem;

    // ---- input loader: unit u < 2 * UNITS -> plane u / UNITS, then (row,
    // 8-pixel group, channel half) as in the dense kernel; thread tid takes
    // units tid and tid + 256
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (int64_t)n * C * HW, (uint32_t)C * HW * 2);
    constexpr int kUnits = 2 * G::UNITS;
    uint32_t ivoff[2], idst[2];
    bool act[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int u = tid + kThreads * k;
        act[k] = u < kUnits;
        const int pl = act[k] ? u / G::UNITS : 0, v = act[k] ? u - pl * G::UNITS : 0;
        const int rho = v % kInRows, rest = v / kInRows;
        const int pg = rest % (W / 8), g8 = rest / (W / 8);
        const int ih = r0 - 1 + rho;
        const bool ok = act[k] && ih >= 0 && ih < H;
        ivoff[k] = ok ? (uint32_t)((((gA + pl) * Cg + g8 * 8) * HW + ih * W + pg * 8) * 2) : kOob;
        idst[k] = (uint32_t)(pl * G::IN_BYTES + (rho * RP + pg * 8 + 1) * kPix + in_half(g8, rho) * 16);
    }
    const uint32_t chan_bytes = (uint32_t)HW * 2, stage_bytes = chan_bytes * kIc;
    uint4 xin[2][8];
    auto load_x = [&](int s) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (k == 1 && kUnits <= kThreads) break;
#pragma unroll
            for (int e = 0; e < 8; ++e) xin[k][e] = bload16(xr, ivoff[k] + e * chan_bytes, (uint32_t)s * stage_bytes);
        }
    };
    auto store_x = [&]() {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (k == 1 && kUnits <= kThreads) break;
            if (!act[k]) continue;
            const uint32_t *v = reinterpret_cast<const uint32_t *>(xin[k]);   // v[e*4 + j/2]: channel e, pixels j, j+1
            uint8_t *dst = ibuf + idst[k];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int dj = j >> 1, hj = j & 1;
                uint4 o;
                o.x = pack_halves(v[0 * 4 + dj], hj, v[1 * 4 + dj], hj);
                o.y = pack_halves(v[2 * 4 + dj], hj, v[3 * 4 + dj], hj);
                o.z = pack_halves(v[4 * 4 + dj], hj, v[5 * 4 + dj], hj);
                o.w = pack_halves(v[6 * 4 + dj], hj, v[7 * 4 + dj], hj);
                *reinterpret_cast<uint4 *>(dst + j * kPix) = o;
            }
        }
    };
    // ---- weights: packed as a layer of Cg input channels
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp + (int64_t)blockIdx.y * kPackOcBlock * Cg * 9,
                                                (uint32_t)kPackOcBlock * Cg * 9 * 2);
    const uint32_t lane16 = (uint32_t)lane * 16;
    auto dma_w = [&](int s) {
        for (int blk = wave; blk < 18; blk += 4) {
            const int tap = blk >> 1, u = blk & 1;
            dma_1k(wlds + tap * kTapBytes + u * 1024, wr, lane16,
                   s * kPackStage + tap * (kPackOcBlock * 32) + half * kTapBytes + u * 1024);
        }
    };

    // operands: A as in the dense kernel; B from this wave row's plane
    const uint32_t a_off = (uint32_t)((wm * 32 + l32) * 32 + ((h ^ wswz(l32)) * 16));
    const int c0 = wn * J;
    const uint32_t pl_off = (uint32_t)(wm * G::IN_BYTES);
    const uint32_t b_base = pl_off + (uint32_t)((((l32 & 7) * RP) + D * (l32 >> 3) + c0) * kPix +
                                                in_half(h, l32 & 7) * 16);
    const uint32_t b1_base = pl_off + (uint32_t)(((((l32 & 7) + 1) * RP) + D * (l32 >> 3) + c0) * kPix +
                                                 in_half(h, (l32 & 7) + 1) * 16);
    const uint32_t b2_base = pl_off + (uint32_t)(((((l32 & 7) + 2) * RP) + D * (l32 >> 3) + c0) * kPix +
                                                 in_half(h, (l32 & 7) + 2) * 16);

    // zero the halo columns of both planes (never written by the loader)
    zero_halo<W, RP, 1>(ibuf, 2, tid);
    const float bv = bias ? bias[ocb + wm * 32 + l32] : 0.f;
    f32x16_t acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = bv;
    __syncthreads();

    for (int s = 0; s < S; ++s) {
        dma_w(s);
        load_x(s);
        CONV3X3_WAIT_VMCNT(0);
        store_x();
        __syncthreads();            // this stage's weights and planes visible
        const uint8_t *wb = wbuf + a_off;
        const uint8_t *ib = ibuf + b_base, *tb = ibuf + b1_base, *ub = ibuf + b2_base;
        uint4 A[9], B0[2], T1[2], T2[2];
#pragma unroll
        for (int tp = 0; tp < 9; ++tp) A[tp] = *reinterpret_cast<const uint4 *>(wb + tp * kTapBytes);
        B0[0] = *reinterpret_cast<const uint4 *>(ib);
        T1[0] = *reinterpret_cast<const uint4 *>(tb);
        T2[0] = *reinterpret_cast<const uint4 *>(ub);
        __builtin_amdgcn_s_setprio(1);
        cg_col<D, 1, 0>(acc, A, B0, T1, T2, ib, tb, ub, [](auto) {});
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();            // buffers free for the next stage
    }

    cg_epilogue<D, OUT, 0, 1>(smem, acc, y, n, Co, ocb, H, r0, relu);
}

// ---------------------------------------------------------------------------
// Persistent variant (NCHW, dilation 1, groups 1): two workgroups per CU, each
// walking a short list of items, instead of one workgroup per tile.
//
// Work units are 32-channel halves of the 64-channel tiles above, numbered
// unit = 2 * tile + half with tile = (image * bands + band) * (C_out / 64) +
// channel block.  CU r (ranked so that the CUs of one XCD take consecutive
// ranges) owns units [r U / NC, (r + 1) U / NC); its two workgroups split the
// range at a tile boundary, so each gets whole tiles plus at most two half
// tiles (a leading one, the upper half of a tile, and a trailing one, the
// lower half).  The workgroup whose unit count is odd starts with a half
// tile and the other with a full one, which puts the two half a tile apart:
// from then on one's epilogue and the next item's prologue (no MFMA work)
// fall into the other's stages instead of coinciding with them.  (Workgroups
// b and b + NC of a grid of two per CU share a CU under the dispatcher's
// placement; the schedule is correct for any placement, only the overlap
// relies on it.)  The unit ranges also even out the work per CU, where one
// workgroup per tile leaves 1.75 rounds of tiles on the 3x3 layer at
// N = 64.
//
// A half tile (32 channels x 8 rows x W) puts its four waves side by side
// over the D fragment columns: ceil(D/4) each for waves 0 and 1, floor(D/4)
// for waves 2 and 3, with the weights of its 32 channels in rows 0 .. 31 of
// each tap.  Between items, the next item's stage-0 weights are copied into
// weight buffer 0 during the last stage (when C_in / 16 is even, that stage
// reads buffer 1), its stage-0 input is loaded into registers halfway
// through the last stage, and the epilogue image lies above weight buffer 0,
// so the only pause between items is the epilogue itself and one wait.
// The epilogue overwrites the input buffers' zero halo columns, so they are
// cleared again before the next item's input goes in.

// The MFMAs of input-fragment column q for a wave of J output fragments.
template <int J, int RR>
__device__ __forceinline__ void cgp_mfma(f32x16_t (&acc)[J], const uint4 (&A)[9], const uint4 &b, int q) {
#pragma unroll
    for (int kw = 0; kw < 3; ++kw) {
        const int j = q - kw;
        if (j >= 0 && j < J) acc[j] = mfma32x32x16(b, A[RR * 3 + kw], acc[j]);
    }
}

// Column step q of a stage (as cg_col, for a wave of J fragments).
template <int J, int q, class Mid>
__device__ __forceinline__ void cgp_col(f32x16_t (&acc)[J], const uint4 (&A)[9], uint4 (&B0)[2], uint4 (&T1)[2],
                                        uint4 (&T2)[2], const uint8_t *ib, const uint8_t *tb, const uint8_t *ub,
                                        Mid &&mid) {
    constexpr int Q = J + 2;
    if constexpr (q + 1 < Q) {
        B0[(q + 1) & 1] = *reinterpret_cast<const uint4 *>(ib + (q + 1) * kPix);
        T1[(q + 1) & 1] = *reinterpret_cast<const uint4 *>(tb + (q + 1) * kPix);
        T2[(q + 1) & 1] = *reinterpret_cast<const uint4 *>(ub + (q + 1) * kPix);
    }
    cgp_mfma<J, 0>(acc, A, B0[q & 1], q);
    cgp_mfma<J, 1>(acc, A, T1[q & 1], q);
    cgp_mfma<J, 2>(acc, A, T2[q & 1], q);
    if constexpr (q == Q / 2) mid();
    if constexpr (q + 1 < Q) cgp_col<J, q + 1>(acc, A, B0, T1, T2, ib, tb, ub, mid);
}

// Epilogue of one item, NCHW: NP passes of 32 channels (2 for a full tile, 1
// for a half tile) through the image at epi, laid out and read back as in
// cg_epilogue; in pass p the waves with wpass == p write their fragments
// (columns c0 .. c0 + J - 1 of each row and column group).  yr covers the
// item's channel planes.
template <int D, int OUT, int J, int NP>
__device__ __forceinline__ void cgp_epilogue(float *epi, const f32x16_t (&acc)[J], __amdgpu_buffer_rsrc_t yr, int HW,
                                             int H, int r0, int relu, int c0, int wpass, int lane) {
    constexpr int W = 4 * D;
    constexpr int P = EpiGeo<W>::P;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    constexpr int kOutB = OUT ? 2 : 4;
    float *const wdst = epi + l32 * P + 4 * h * W + c0;
    constexpr int kF = OUT ? 4 : 2;
    constexpr int kU = kRows * W / kF;
    constexpr int kIt = (kU + 63) / 64;
    uint32_t voff[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int u = lane + 64 * it, e = u * kF;
        const int row = e / W, col = e - row * W, orow = r0 + row;
        voff[it] = (u < kU && orow < H) ? (uint32_t)((orow * W + col) * kOutB) : kOob;
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        if (wpass == p) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float *base = wdst + (r & 3) * W + (r >> 2) * D;
#pragma unroll
                for (int j = 0; j < J; ++j) base[j] = acc[j][r];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        auto readback = [&](auto rc) {
            constexpr bool R = decltype(rc)::value;
#pragma unroll
            for (int i = 0; i < kEpiOc / 4; ++i) {
                const int c = wave * (kEpiOc / 4) + i;
                const float *src = epi + c * P + lane * kF;
                const uint32_t soff = (uint32_t)((p * kEpiOc + c) * HW * kOutB);
#pragma unroll
                for (int it = 0; it < kIt; ++it) {
                    float f[4];
                    const float2 a = *reinterpret_cast<const float2 *>(src + it * 64 * kF);
                    f[0] = a.x; f[1] = a.y;
                    if (OUT) {
                        const float2 b = *reinterpret_cast<const float2 *>(src + it * 64 * kF + 2);
                        f[2] = b.x; f[3] = b.y;
                    }
                    u32x2_t va;
                    if (OUT == 0) {
                        va[0] = __float_as_uint(R ? fmaxf(f[0], 0.f) : f[0]);
                        va[1] = __float_as_uint(R ? fmaxf(f[1], 0.f) : f[1]);
                    } else {
                        uint32_t b[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) b[u] = f32_to_bf16_rne(R ? fmaxf(f[u], 0.f) : f[u]);
                        va[0] = b[0] | (b[1] << 16);
                        va[1] = b[2] | (b[3] << 16);
                    }
                    __builtin_amdgcn_raw_buffer_store_b64(va, yr, (int)voff[it], (int)soff, 0);
                }
            }
        };
        if (relu) readback(BoolC<true>{}); else readback(BoolC<false>{});
        if (p + 1 < NP) __syncthreads();
    }
}

// LDS of the persistent kernel: weight buffers 0 and 1, input buffers 0 and
// 1, and the epilogue image from EPI on (above weight buffer 0 when that fits
// in 80 KB, so that the next item's first weights survive the epilogue).
template <int D>
struct CgpGeo {
    using G = Geo<D, 1>;
    static constexpr int STAGES = 2 * kWStage + 2 * G::IN_BYTES;
    static constexpr int EPI = kWStage + EpiGeo<G::W>::BYTES <= 80 * 1024 ? kWStage : 0;
    static constexpr int LDS = STAGES > EPI + EpiGeo<G::W>::BYTES ? STAGES : EPI + EpiGeo<G::W>::BYTES;
};

template <int D, int OUT>
__global__ __launch_bounds__(kThreads, 2)
void conv3x3cgp_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wp,
                       const float *__restrict__ bias, float *__restrict__ y,
                       int C, int H, int Co, int rb_per_img, int units, int relu) {
    using G = Geo<D, 1>;
    using CG = CgpGeo<D>;
    constexpr int W = G::W, RP = G::RP;
    constexpr int JF = D / 2, JH = (D + 3) / 4, JL = D / 4;   // fragments per wave: full tile; half tile waves 0-1, 2-3
    static_assert(2 * JH + 2 * JL == D, "D is even");
    __shared__ __align__(16) uint8_t smem[CG::LDS];
    static_assert(CG::LDS <= 80 * 1024, "two workgroups per CU");

    // ---- this workgroup's units [u0, u1)
    const int NC = (int)gridDim.x >> 1;
    const int slot = (int)blockIdx.x >= NC, cu = (int)blockIdx.x - slot * NC;
    const int rank = (NC % 8 == 0) ? (cu & 7) * (NC >> 3) + (cu >> 3) : cu;
    const int h0 = (int)((int64_t)rank * units / NC), h1 = (int)((int64_t)(rank + 1) * units / NC);
    const int hh = h1 - h0;
    const int mid_u = h0 + hh / 2;
    const int split = ((hh & 1) && (mid_u & 1)) ? mid_u + 1 : mid_u;   // a tile boundary when hh is odd
    const int u0 = slot ? split : h0, u1 = slot ? h1 : split;
    if (u0 >= u1) return;                                  // uniform: no barrier is reached
    const int nA = split - h0, nB = h1 - split;
    const bool a_half_first = (nA & 1) && !(nB & 1);
    const int lead = u0 & 1, trail = u1 & 1;               // upper half of tile u0/2; lower half of tile (u1-1)/2
    const int f0 = (u0 + 1) >> 1, f1 = u1 >> 1;
    const int nf = f1 > f0 ? f1 - f0 : 0;
    const bool half_first = slot ? ((lead | trail) && !a_half_first) : a_half_first;
    const int n_items = lead + nf + trail;
    // item i -> (tile, sub): sub -1 a full tile, 0 / 1 its lower / upper 32 channels
    auto item = [&](int i, int &tile, int &sub) {
        if (half_first) {
            if (i == 0) {
                if (lead) { tile = u0 >> 1; sub = 1; } else { tile = (u1 - 1) >> 1; sub = 0; }
                return;
            }
            --i;
            if (i < nf) { tile = f0 + i; sub = -1; return; }
            tile = (u1 - 1) >> 1; sub = 0;                 // the trail, after a lead taken first
            return;
        }
        if (i < nf) { tile = f0 + i; sub = -1; return; }
        i -= nf;
        if (lead && i == 0) { tile = u0 >> 1; sub = 1; return; }
        tile = (u1 - 1) >> 1; sub = 0;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int HW = H * W;
    const int S = C / kIc;
    const int NO = Co / kOc;                               // 64-channel blocks
    uint8_t *const wbuf = smem;
    uint8_t *const ibuf = smem + 2 * kWStage;
    lds_u8 *const wlds = (lds_u8 *)smem;
    float *const epi = reinterpret_cast<float *>(smem + CG::EPI);
    constexpr bool kPreW = CG::EPI > 0;                    // weight buffer 0 survives the epilogue
    const bool pre_w = kPreW && (S & 1) == 0;              // ... and the last stage leaves it free

    // ---- per-item state: image, first row, first channel, 64-channel block
    struct It {
        int n, r0, ocb, o, half;
    };
    const bool in_active = tid < G::UNITS;
    const bool x_wave = wave * 64 < G::UNITS;   // this wave has lanes that own units (and issues their loads)
    const int rho = tid % kInRows, rest = tid / kInRows;
    const int pg = rest % (W / 8), g8 = in_active ? rest / (W / 8) : 0;
    const uint32_t idst = (uint32_t)((rho * RP + pg * 8 + 1) * kPix + in_half(g8, rho) * 16);
    const uint32_t chan_bytes = (uint32_t)HW * 2, stage_bytes = chan_bytes * kIc;
    const uint32_t lane_x = (uint32_t)((g8 * 8 * HW + pg * 8) * 2);
    auto make_item = [&](int i, It &it) {
        int tile, sub;
        item(i, tile, sub);
        const int nb = tile / NO;
        it.o = tile - nb * NO;
        it.n = nb / rb_per_img;
        it.r0 = (nb - it.n * rb_per_img) * kRows;
        it.half = sub >= 0;
        it.ocb = it.o * kOc + (sub > 0 ? 32 : 0);
    };
    uint4 xin[8];
    // stage s of image n, rows r0 - 1 .. r0 + 8 (one call site per phase, so
    // that the loaded registers are never merged across branches, which
    // would need a wait for the loads)
    auto load_x = [&](int n, int r0, int s) {
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (int64_t)n * C * HW, (uint32_t)C * HW * 2);
        const int ih = r0 - 1 + rho;
        const uint32_t ivoff = (ih >= 0 && ih < H) ? lane_x + (uint32_t)(ih * W * 2) : kOob;
        if (!in_active) return;              // as in the one-tile kernel: idle lanes issue nothing
#pragma unroll
        for (int e = 0; e < 8; ++e) xin[e] = bload16(xr, ivoff + e * chan_bytes, (uint32_t)s * stage_bytes);
    };
    auto store_x = [&](int buf) {
        if (!in_active) return;
        const uint32_t *v = reinterpret_cast<const uint32_t *>(xin);   // v[e*4 + j/2]: channel e, pixels j, j+1
        uint8_t *dst = ibuf + buf * G::IN_BYTES + idst;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int dj = j >> 1, hj = j & 1;
            uint4 o;
            o.x = pack_halves(v[0 * 4 + dj], hj, v[1 * 4 + dj], hj);
            o.y = pack_halves(v[2 * 4 + dj], hj, v[3 * 4 + dj], hj);
            o.z = pack_halves(v[4 * 4 + dj], hj, v[5 * 4 + dj], hj);
            o.w = pack_halves(v[6 * 4 + dj], hj, v[7 * 4 + dj], hj);
            *reinterpret_cast<uint4 *>(dst + j * kPix) = o;
        }
    };
    // weights of stage s into buffer buf: a full tile copies rows 0 .. 63 of
    // each tap (18 KB), a half tile its 32 rows into rows 0 .. 31 (9 KB)
    const uint32_t lane16 = (uint32_t)lane * 16;
    auto dma_w = [&](const It &it, int s, int buf) {
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(wp + (int64_t)(it.o >> 1) * kPackOcBlock * C * 9,
                                                    (uint32_t)kPackOcBlock * C * 9 * 2);
        const int woff = (it.o & 1) * kTapBytes + (it.ocb & 32 ? 1024 : 0);
        if (!it.half) {
            for (int blk = wave; blk < 18; blk += 4) {
                const int tap = blk >> 1, u = blk & 1;
                dma_1k(wlds + buf * kWStage + tap * kTapBytes + u * 1024, wr, lane16,
                       s * kPackStage + tap * (kPackOcBlock * 32) + woff + u * 1024);
            }
        } else {
            for (int tap = wave; tap < 9; tap += 4)
                dma_1k(wlds + buf * kWStage + tap * kTapBytes, wr, lane16,
                       s * kPackStage + tap * (kPackOcBlock * 32) + woff);
        }
    };

    // this lane's bias for an item: channel ocb + l32 of its wave row.  The
    // 32 values of the wave row are read with scalar loads (their own
    // counter), so that waiting for them never waits for the input loads in
    // flight, and each lane picks its own.
    auto bias_of = [&](const It &it) {
        float v = 0.f;
        if (bias) {
            const float *bp = bias + it.ocb + (it.half ? 0 : (wave >> 1) * 32);
            const int l32 = lane & 31;
#pragma unroll
            for (int i = 0; i < 32; ++i) v = l32 == i ? bp[i] : v;
        }
        return v;
    };
    It cur, nxt;
    make_item(0, cur);
    zero_halo<W, RP, 1>(ibuf, 2, tid);
    dma_w(cur, 0, 0);
    load_x(cur.n, cur.r0, 0);
    CONV3X3_WAIT_VMCNT(0);
    store_x(0);
    __syncthreads();

    for (int i = 0; i < n_items; ++i) {
        const bool has_next = i + 1 < n_items;
        if (has_next) make_item(i + 1, nxt);
        // one item with J fragments a wave and NP epilogue passes
        auto run = [&](auto jc, auto npc, int arow, int c0, int wpass) {
            constexpr int J = decltype(jc)::value;
            constexpr int NP = decltype(npc)::value;
            // the lane index, opaque to the compiler, so that the per-lane
            // addresses below are computed per item instead of being hoisted
            // out of the item loop for all three item shapes at once (which
            // would not fit in the registers)
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int l32 = ln & 31, h = ln >> 5;
            const uint32_t a_off = (uint32_t)((arow + l32) * 32 + ((h ^ wswz(l32)) * 16));
            const uint32_t b_base = (uint32_t)((((l32 & 7) * RP) + D * (l32 >> 3) + c0) * kPix +
                                               in_half(h, l32 & 7) * 16);
            const uint32_t b1_base = (uint32_t)(((((l32 & 7) + 1) * RP) + D * (l32 >> 3) + c0) * kPix +
                                                in_half(h, (l32 & 7) + 1) * 16);
            const uint32_t b2_base = (uint32_t)(((((l32 & 7) + 2) * RP) + D * (l32 >> 3) + c0) * kPix +
                                                in_half(h, (l32 & 7) + 2) * 16);
            // stage 1's input is loaded here, inside each item shape's code,
            // so that its registers stay those of the loop's own loads (a
            // load before the branch would be copied into them, which needs
            // a wait for it).  Unconditionally (stage 0 again when there is
            // no stage 1, never stored), so that the bias needs no wait for
            // these loads.
            const float bv = bias_of(cur);
            load_x(cur.n, cur.r0, S > 1 ? 1 : 0);
            f32x16_t acc[J];
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][r] = bv;
            for (int s = 0; s < S; ++s) {
                const int b = s & 1;
                const bool more = s + 1 < S;
                const uint8_t *wb = wbuf + b * kWStage + a_off;
                const uint8_t *ib = ibuf + b * G::IN_BYTES + b_base;
                const uint8_t *tb = ibuf + b * G::IN_BYTES + b1_base;
                const uint8_t *ub = ibuf + b * G::IN_BYTES + b2_base;
                uint4 A[9], B0[2], T1[2], T2[2];
#pragma unroll
                for (int t = 0; t < 9; ++t) A[t] = *reinterpret_cast<const uint4 *>(wb + t * kTapBytes);
                B0[0] = *reinterpret_cast<const uint4 *>(ib);
                T1[0] = *reinterpret_cast<const uint4 *>(tb);
                T2[0] = *reinterpret_cast<const uint4 *>(ub);
                // as in the one-tile kernel: the input stored at the middle,
                // then the next weights copied and the input after loaded;
                // the copies are waited for before the barrier
                // (the wait is unconditional, so that the compiler sees no
                // load pending into the input registers past this point)
                auto mid = [&]() {
                    CONV3X3_WAIT_VMCNT(0);
                    if (more) {
                        store_x(b ^ 1);
                        dma_w(cur, s + 1, b ^ 1);
                    } else if (has_next && pre_w) {
                        dma_w(nxt, 0, 0);          // buffer 0: this last stage reads buffer 1
                    }
                    // the input of stage s + 2, or at the last stage the next item's stage 0
                    if (more ? s + 2 < S : has_next)
                        load_x(more ? cur.n : nxt.n, more ? cur.r0 : nxt.r0, more ? s + 2 : 0);
                };
                __builtin_amdgcn_s_setprio(1);
                cgp_col<J, 0>(acc, A, B0, T1, T2, ib, tb, ub, mid);
                __builtin_amdgcn_s_setprio(0);
                if (more) {
                    if (s + 2 < S && x_wave) CONV3X3_WAIT_VMCNT(8);
                    else CONV3X3_WAIT_VMCNT(0);
                }
                __syncthreads();
            }
            const int nch = NP * kEpiOc;
            constexpr int kOutB = OUT ? 2 : 4;
            const __amdgpu_buffer_rsrc_t yr =
                make_rsrc((char *)y + ((int64_t)cur.n * Co + cur.ocb) * HW * kOutB, (uint32_t)nch * HW * kOutB);
            cgp_epilogue<D, OUT, J, NP>(epi, acc, yr, HW, H, cur.r0, relu, c0, wpass, ln);
        };
        if (!cur.half) {
            run(IntC<JF>{}, IntC<2>{}, (wave >> 1) * 32, (wave & 1) * JF, wave >> 1);
        } else if (wave < 2) {
            run(IntC<JH>{}, IntC<1>{}, 0, wave * JH, 0);
        } else {
            run(IntC<JL>{}, IntC<1>{}, 0, 2 * JH + (wave - 2) * JL, 0);
        }
        if (has_next) {
            __syncthreads();                   // the epilogue image is read; its space is stage space again
            zero_halo<W, RP, 1>(ibuf, 2, tid);
            if (!pre_w) dma_w(nxt, 0, 0);
            CONV3X3_WAIT_VMCNT(0);
            store_x(0);
            __syncthreads();
            cur = nxt;
        }
    }
}

}  // namespace

bool conv3x3cg_supported(const Shape &sh, const void *x, const void *w) {
    (void)w;
    const int64_t HW = (int64_t)sh.H * sh.W;
    const int dl = sh.dil;
    const bool grouped_pair = sh.G > 1 && sh.Cog() == 32 && sh.Cg() % kIc == 0 && dl == 1 && !sh.nhwc;
    return (sh.G == 1 || grouped_pair) && (dl == 1 || dl == 2) && sh.ndim == 2 && sh.K == 3 && sh.s == 1 &&
           sh.p == dl && sh.Cg() % kIc == 0 &&
           sh.Co % kPackOcBlock == 0 && sh.W % 8 == 0 && sh.W >= 32 && sh.W <= 64 &&
           (int64_t)sh.C * HW * 2 < (INT64_C(1) << 31) &&                 // one image within a buffer range
           (int64_t)kOc * HW * 4 < (INT64_C(1) << 31) &&                  // one output block within a buffer range
           (!sh.nhwc || HW * sh.Co * 4 < (INT64_C(1) << 31)) &&           // channels-last: one output image
           (int64_t)kPackOcBlock * sh.Cg() * 9 * 2 < (INT64_C(1) << 31) &&
           (int64_t)sh.N * dl * ((sh.H + kRows * dl - 1) / (kRows * dl)) * 2 < (INT64_C(1) << 31) &&
           ((uintptr_t)x % 16) == 0;
}

// The persistent variant: NCHW, dilation 1, groups 1, and a unit count
// (two per 64-channel tile) that fits an int.
bool conv3x3cgp_supported(const Shape &sh, const void *x, const void *w) {
    const int64_t rb = (sh.H + kRows - 1) / kRows;
    return conv3x3cg_supported(sh, x, w) && sh.G == 1 && sh.dil == 1 && !sh.nhwc &&
           (int64_t)sh.N * rb * (sh.Co / kOc) * 2 < (INT64_C(1) << 31);
}

namespace {
// CU count of the current device, per host thread (0 if it cannot be read).
int cu_count() {
    thread_local int cached_dev = -1, num_cu = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev != cached_dev) {
        int n = 0;
        num_cu = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 0;
        cached_dev = dev;
    }
    return num_cu;
}
}  // namespace

// Whether to run the persistent kernel rather than one workgroup per tile.
// Measured on the 3x3 layer (C = 128, 56 x 56): its half tiles take nearly
// as long as whole tiles (the input staging, not the matrix cores, sets a
// stage's time), so it wins only while the layer has no more 32-channel
// units than the device has CUs and one workgroup per tile would leave CUs
// idle (N = 8: 17.2 against 19.7 us; N = 16: 23.3 against 21.1; N = 64:
// 4% slower).  CONVFWD_3X3_PERSISTENT=1 or 0 forces the choice either way.
bool conv3x3cgp_preferred(const Shape &sh) {
    const char *e = getenv("CONVFWD_3X3_PERSISTENT");
    if (e && e[0] == '1') return true;
    if (e && e[0] == '0') return false;
    const int64_t units = (int64_t)sh.N * ((sh.H + kRows - 1) / kRows) * (sh.Co / kOc) * 2;
    const int ncu = cu_count();
    return ncu > 0 && units <= ncu;
}

hipError_t launch_conv3x3cgp_bf16(const Shape &sh, const uint16_t *x, const uint16_t *wpack, const float *bias,
                                  float *y, hipStream_t st) {
    int num_cu = cu_count();
    if (num_cu <= 0) num_cu = 256;
    const int rb = (sh.H + kRows - 1) / kRows;
    const int units = sh.N * rb * (sh.Co / kOc) * 2;
    const dim3 grid((unsigned)(2 * num_cu));
#define CONV3X3CGP_GO(DV)                                                                                     \
    if (sh.out_bf16)                                                                                          \
        hipLaunchKernelGGL((conv3x3cgp_kernel<DV, 1>), grid, dim3(kThreads), 0, st, x, wpack, bias, y, sh.C,    \
                           sh.H, sh.Co, rb, units, sh.relu);                                                  \
    else                                                                                                      \
        hipLaunchKernelGGL((conv3x3cgp_kernel<DV, 0>), grid, dim3(kThreads), 0, st, x, wpack, bias, y, sh.C,    \
                           sh.H, sh.Co, rb, units, sh.relu)
    switch (sh.W / 4) {
        case 8: CONV3X3CGP_GO(8); break;
        case 10: CONV3X3CGP_GO(10); break;
        case 12: CONV3X3CGP_GO(12); break;
        case 14: CONV3X3CGP_GO(14); break;
        case 16: CONV3X3CGP_GO(16); break;
        default: return hipErrorInvalidValue;
    }
#undef CONV3X3CGP_GO
    return hipGetLastError();
}

hipError_t launch_conv3x3cg_bf16(const Shape &sh, const uint16_t *x, const uint16_t *wpack, const float *bias,
                                 float *y, hipStream_t st) {
    const int dl = sh.dil;                               // 1 or 2 (conv3x3cg_supported)
    const int rb = dl * ((sh.H + kRows * dl - 1) / (kRows * dl));   // tiles per image: bands x row phases
    const int64_t blocks = (int64_t)sh.N * rb * 2;       // tiles x two 64-channel halves
    const int remap = (blocks % 8 == 0) ? 1 : 0;
    dim3 grid((unsigned)blocks, (unsigned)(sh.Co / kPackOcBlock));
#define CONV3X3CG_GO(DV, O, L)                                                                                 \
    if (dl == 1)                                                                                                \
        hipLaunchKernelGGL((conv3x3cg_kernel<DV, O, L, 1>), grid, dim3(kThreads), 0, st, x, wpack, bias, y, sh.C,  \
                           sh.H, sh.Co, rb, remap, sh.relu);                                                    \
    else                                                                                                        \
        hipLaunchKernelGGL((conv3x3cg_kernel<DV, O, L, 2>), grid, dim3(kThreads), 0, st, x, wpack, bias, y, sh.C,  \
                           sh.H, sh.Co, rb, remap, sh.relu)
#define CONV3X3CG_LAUNCH(DV)                                              \
    if (sh.nhwc) {                                                        \
        if (sh.out_bf16) CONV3X3CG_GO(DV, 1, 1); else CONV3X3CG_GO(DV, 0, 1); \
    } else {                                                              \
        if (sh.out_bf16) CONV3X3CG_GO(DV, 1, 0); else CONV3X3CG_GO(DV, 0, 0); \
    }
    if (sh.G > 1) {
#define CONV3X3CG_GP(DV)                                                                                    \
    if (sh.out_bf16)                                                                                        \
        hipLaunchKernelGGL((conv3x3cg_gp_kernel<DV, 1>), grid, dim3(kThreads), 0, st, x, wpack, bias, y, sh.C, \
                           sh.H, sh.Co, sh.Cg(), rb, remap, sh.relu);                                      \
    else                                                                                                    \
        hipLaunchKernelGGL((conv3x3cg_gp_kernel<DV, 0>), grid, dim3(kThreads), 0, st, x, wpack, bias, y, sh.C, \
                           sh.H, sh.Co, sh.Cg(), rb, remap, sh.relu)
        switch (sh.W / 4) {
            case 8: CONV3X3CG_GP(8); break;
            case 10: CONV3X3CG_GP(10); break;
            case 12: CONV3X3CG_GP(12); break;
            case 14: CONV3X3CG_GP(14); break;
            case 16: CONV3X3CG_GP(16); break;
            default: return hipErrorInvalidValue;
        }
#undef CONV3X3CG_GP
        return hipGetLastError();
    }
    switch (sh.W / 4) {
        case 8: CONV3X3CG_LAUNCH(8); break;
        case 10: CONV3X3CG_LAUNCH(10); break;
        case 12: CONV3X3CG_LAUNCH(12); break;
        case 14: CONV3X3CG_LAUNCH(14); break;
        case 16: CONV3X3CG_LAUNCH(16); break;
        default: return hipErrorInvalidValue;
    }
#undef CONV3X3CG_LAUNCH
#undef CONV3X3CG_GO
    return hipGetLastError();
}

}  // namespace convfwd
