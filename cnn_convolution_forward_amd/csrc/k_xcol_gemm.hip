// k_xcol_gemm.hip -- the explicit route's GEMM, Y = W_row @ X_col, with X_col
// already written to HBM by the im2col kernel ("Why use matrix multiplication
// for convolution", 2.3 and 3.2: the patch matrix times the flattened
// kernels, then the reshape to NCHW).
//
// X_col has C_in*K^d rows of J = N*out_plane columns (the pixels of all images
// side by side), so this is one plain GEMM with a tiny M (C_out) and a huge N:
// every X_col byte is read exactly once, and the layer streams K^d times the
// input's bytes.  Both operands travel global -> LDS by direct-to-LDS loads
// (no registers, no VALU work) into a ring of NS stage buffers, NS - 1 stages
// ahead of the MFMAs.  On the 3x3 layer (462 MB of X_col) this takes 148 us
// by events (160 us, the rocprofv3 median) against 187 us on the tiled
// pointwise kernel, which loads one stage ahead through registers.  A deeper
// ring (4 or 5 stages) did not help, and a build without the output stores
// took 129 us (X_col read at ~3.6 TB/s).
//
// Tile: 128 output channels x up to TN = 256 pixels (8 columns of 32), four
// waves in a 2 x 2 grid, each 2 x 4 v_mfma_f32_32x32x16_bf16 tiles (64 x 128).
// A stage is 32 reduction rows: A [oc 128][k 32] (64-byte rows, 16-byte quads
// swizzled by bits 2-3 of the row, so a fragment read of 16 consecutive rows
// hits 16 distinct bank groups) and B [k 32][px TN] (16-byte units swizzled
// by 4 * (k % 4), so the four rows of a transposing read start on different
// bank groups).  Three stage buffers (72 KB): two workgroups per CU, each
// with two stages in flight.  The swizzles are applied on the global side:
// each lane of a direct-to-LDS load picks the global 16 bytes that belong at
// its fixed LDS slot.  B fragments come from ds_read_b64_tr_b16 transposing
// reads (pixels contiguous in X_col, the operand wants 8 consecutive k per
// pixel).
//
// Epilogue: accumulators start at the bias; fp32 (or bf16) stores from the
// accumulators, 32 lanes on 32 consecutive pixels of one channel (y is NCHW:
// pixel px of X_col is image px / plane, position px % plane).
//
// Requirements (checked by the launcher): groups 1, NCHW, C_in*K^d % 32 == 0,
// J % 8 == 0, X_col, W_row and y below 2 GiB, 16-byte aligned X_col and w.
#include "conv_internal.h"
#include "conv3x3_common.h"

namespace convfwd {
namespace {

constexpr int kXM = 128, kXK = 32;
constexpr int kAStage = kXM * kXK * 2;            // 8 KB

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ uint2 xg_read_tr(const uint8_t *p) {
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p));
    return __builtin_bit_cast(uint2, v);
}

// LDS slot (16-byte unit) of A quad q (k = 8q .. 8q+7) of tile row m
__device__ __forceinline__ int a_slot(int m, int q) { return m * 4 + (q ^ ((m >> 2) & 3)); }
// LDS byte of B element (k, px) inside a stage's B image (TN pixels a row)
template <int TN>
__device__ __forceinline__ int b_byte(int k, int px) {
    return (k * (TN / 8) + ((px >> 3) ^ (4 * (k & 3)))) * 16 + (px & 7) * 2;
}

// stage waits: this wave issued PER direct-to-LDS loads per stage; `ahead`
// stages after the one about to be read may stay in flight
template <int PER>
__device__ __forceinline__ void wait_ahead(int ahead) {
    if (ahead >= 4) CONV3X3_WAIT_VMCNT(4 * PER);
    else if (ahead == 3) CONV3X3_WAIT_VMCNT(3 * PER);
    else if (ahead == 2) CONV3X3_WAIT_VMCNT(2 * PER);
    else if (ahead == 1) CONV3X3_WAIT_VMCNT(PER);
    else CONV3X3_WAIT_VMCNT(0);
}

template <int NS, int TN>
__global__ __launch_bounds__(256, 2)
void xcol_gemm_kernel(const uint16_t *__restrict__ xcol, const uint16_t *__restrict__ w,
                      const float *__restrict__ bias, float *__restrict__ y,
                      int K, int Co, int plane, int J, int NC, int NR, int ncb, int remap, int out_bf16, int relu) {
    constexpr int kBStage = kXK * TN * 2;          // 16 KB at TN = 256
    constexpr int kStage = kAStage + kBStage;
    constexpr int TC = TN / 32;                    // 32-pixel columns per full tile
    constexpr int JT = TN / 64;                    // 32-pixel MFMA tiles per wave
    constexpr int BC = TN / 64;                    // B chunks (1 KB) per wave per stage
    constexpr int PER = 2 + BC;                    // direct-to-LDS loads per wave per stage
    static_assert(NS >= 2 && NS <= 5 && NS * kStage <= 80 * 1024, "two workgroups per CU");
    __shared__ __align__(16) uint8_t smem[NS * kStage];
    lds_u8 *const lds = (lds_u8 *)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // block -> (channel block ob, column range r): the NC 32-pixel columns
    // are split into NR contiguous ranges of floor or ceil(NC / NR) columns,
    // walked in tiles of at most TC columns.  The launcher makes each range
    // one tile; 512 workgroups walking two or three tiles each (no partly
    // filled last round) measured slower on the 3x3 layer (157 against 148 us).
    // With remap, XCD x (block b runs on XCD b % 8) takes the contiguous
    // logical range [x T/8, (x+1) T/8), so the ncb channel blocks of a column
    // range share one XCD's L2 and read their X_col tile from HBM once
    const int T = NR * ncb;
    int L = (int)blockIdx.x;
    if (remap) L = (L & 7) * (T >> 3) + (L >> 3);
    const int ob = L % ncb, r = L / ncb;
    const int c_begin = (int)((int64_t)r * NC / NR), c_end = (int)((int64_t)(r + 1) * NC / NR);
    const int m0 = ob * kXM;
    const int S = K / kXK;

    const __amdgpu_buffer_rsrc_t ar = make_rsrc(w, (uint32_t)Co * (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(xcol, (uint32_t)K * (uint32_t)J * 2u);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)((int64_t)J * Co * (out_bf16 ? 2 : 4)));
    // a resource with no records reads 0: no bias, and rows past C_out
    const __amdgpu_buffer_rsrc_t biasr = make_rsrc(bias ? (const void *)bias : (const void *)w,
                                                   bias ? (uint32_t)Co * 4u : 0u);

    // direct-to-LDS sources: wave w fills A chunks 2w, 2w+1 and B chunks
    // BC w .. BC w + BC - 1 (1 KB each, 64 lanes x 16 bytes, lane l at chunk
    // byte 16 l).  Rows past C_out read row 0 instead, and pixel units past
    // the tile (or past J) read the tile's first unit: a GEMM row (column)
    // depends only on its own A row (B column), those outputs are never
    // stored, and lanes reading one address share one cache line.
    uint32_t a_vo[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int s = (2 * wave + c) * 64 + lane;
        const int m = s >> 2, qs = s & 3;
        const int q = qs ^ ((m >> 2) & 3);
        const int row = m0 + m < Co ? m0 + m : 0;
        a_vo[c] = (uint32_t)(row * K + q * 8) * 2u;
    }
    int b_k[BC], b_u[BC];
#pragma unroll
    for (int c = 0; c < BC; ++c) {
        const int s = (BC * wave + c) * 64 + lane;
        b_k[c] = s / (TN / 8);
        b_u[c] = (s % (TN / 8)) ^ (4 * (b_k[c] & 3));
    }
    const uint32_t b_kstep = (uint32_t)kXK * (uint32_t)J * 2u;

    // fragment reads (byte offsets inside a stage buffer)
    uint32_t a_rd[2][2], b_lo[2][JT], b_hi[2][JT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < 2; ++i) a_rd[kk][i] = (uint32_t)a_slot(wm * 64 + i * 32 + (lane & 31), kk * 2 + (lane >> 5)) * 16u;
        const int kr = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int px = wn * (TN / 2) + j * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            b_lo[kk][j] = (uint32_t)(kAStage + b_byte<TN>(kr, px));
            b_hi[kk][j] = (uint32_t)(kAStage + b_byte<TN>(kr + 4, px));
        }
    }
    float bv[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            bv[i][q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                biasr, (m0 + wm * 64 + i * 32 + mfma32_row(q, lane)) * 4, 0, 0));

    for (int c0 = c_begin; c0 < c_end; c0 += TC) {
        const int cw = c_end - c0 < TC ? c_end - c0 : TC;      // columns in this tile
        const int px0 = c0 * 32;
        uint32_t b_vo[BC];
#pragma unroll
        for (int c = 0; c < BC; ++c) {
            const int px = px0 + 8 * b_u[c];
            const int pxc = (b_u[c] < 4 * cw && px < J) ? px : px0;
            b_vo[c] = ((uint32_t)b_k[c] * (uint32_t)J + (uint32_t)pxc) * 2u;
        }
        auto dma = [&](int kt) {
            lds_u8 *base = lds + (kt % NS) * kStage;
#pragma unroll
            for (int c = 0; c < 2; ++c) dma_1k(base + (2 * wave + c) * 1024, ar, a_vo[c], kt * kXK * 2);
#pragma unroll
            for (int c = 0; c < BC; ++c)
                dma_1k(base + kAStage + (BC * wave + c) * 1024, br, b_vo[c], (int)(kt * b_kstep));
        };

        f32x16_t acc[2][JT];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < JT; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = bv[i][q];

        // every wave's reads of the previous tile's buffers are over (and the
        // compiler's own wait for the bias loads, which does not count the
        // copies, is behind us)
        CONV3X3_WAIT_VMCNT(0);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < S) dma(s);

        for (int kt = 0; kt < S; ++kt) {
            // this wave's copies of stage kt have landed; every wave's are
            // visible after the barrier, which also ends every wave's reads of
            // stage kt - 1 (whose buffer the copy issued next refills)
            const int ahead = S - 1 - kt < NS - 2 ? S - 1 - kt : NS - 2;
            wait_ahead<PER>(ahead);
            __syncthreads();
            if (kt + NS - 1 < S) dma(kt + NS - 1);
            const uint8_t *st = smem + (kt % NS) * kStage;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint4 a[2], b[JT];
#pragma unroll
                for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const uint4 *>(st + a_rd[kk][i]);
#pragma unroll
                for (int j = 0; j < JT; ++j) {
                    const uint2 lo = xg_read_tr(st + b_lo[kk][j]);
                    const uint2 hi = xg_read_tr(st + b_hi[kk][j]);
                    b[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < JT; ++j)
                        if (wn * JT + j < cw) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
            }
        }

        // epilogue: lane l holds pixel px (fixed per j) of 16 channel rows a tile
        uint32_t base[JT];
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int px = px0 + wn * (TN / 2) + j * 32 + (lane & 31);
            const int n = px / plane, q = px - n * plane;
            base[j] = (px < J && wn * JT + j < cw) ? (uint32_t)((int64_t)n * Co * plane + q) : kOob;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int oc = m0 + wm * 64 + i * 32 + mfma32_row(q, lane);
#pragma unroll
                for (int j = 0; j < JT; ++j) {
                    const bool ok = oc < Co && base[j] != kOob;
                    const uint32_t e = base[j] + (uint32_t)oc * (uint32_t)plane;   // element index
                    float v = acc[i][j][q];
                    if (relu) v = fmaxf(v, 0.f);
                    if (out_bf16)
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(v), yr,
                                                              (int)(ok ? e * 2u : kOob), 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yr, (int)(ok ? e * 4u : kOob), 0, 0);
                }
            }
    }
}

}  // namespace

bool gemm_xcol_dma_supported(const Shape &sh, const void *xcol, const void *w) {
    const int64_t rows = sh.xcol_rows(), J = sh.pixels();
    const int64_t ybytes = sh.y_elems() * (sh.out_bf16 ? 2 : 4);
    return sh.G == 1 && !sh.nhwc && rows % kXK == 0 && J % 8 == 0 && rows * J * 2 < (INT64_C(1) << 31) &&
           (int64_t)sh.Co * rows * 2 < (INT64_C(1) << 31) && ybytes < (INT64_C(1) << 31) &&
           ((uintptr_t)xcol % 16) == 0 && ((uintptr_t)w % 16) == 0;
}

hipError_t launch_gemm_xcol_dma_bf16(const Shape &sh, const uint16_t *w, const uint16_t *xcol, const float *bias,
                                     float *y, hipStream_t st) {
    constexpr int kNS = 3, kTN = 256;
    const int J = (int)sh.pixels();
    const int ncb = (sh.Co + kXM - 1) / kXM;
    const int NC = (J + 31) / 32;
    // one range of at most kTN / 32 columns per workgroup (ranges balanced
    // when NC is not a multiple of 8)
    const int NR = (NC + kTN / 32 - 1) / (kTN / 32);
    const int remap = (ncb > 1 && (NR * ncb) % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((xcol_gemm_kernel<kNS, kTN>), dim3((unsigned)(NR * ncb)), dim3(256), 0, st, xcol, w, bias, y,
                       (int)sh.xcol_rows(), sh.Co, (int)sh.out_plane(), J, NC, NR, ncb, remap, sh.out_bf16, sh.relu);
    return hipGetLastError();
}

}  // namespace convfwd
