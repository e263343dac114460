// k_conv3x3.hip -- implicit-GEMM convolution for 3x3 kernels, stride 1, pad 1,
// bf16 in, fp32 accumulate and out, on the gfx950 matrix cores.
//
// Same product as the general kernel, Y = W_row @ X_col ("Why use matrix
// multiplication for convolution", 2.3), but the K dimension is ordered
// (ic-chunk, tap, ic) instead of (ic, tap): for a chunk of 16 input channels
// the workgroup stages ONE halo tile of the input in LDS and all nine taps read
// it at shifted addresses, so each input element crosses from memory to LDS
// once per chunk and feeds nine MFMA steps (the page's per-tile unfold that is
// discarded after the multiply, "Hand-writing Conv2D", 4.1 -- here the unfold
// is only an address offset).  The zero padding is materialised in LDS (edge
// columns and out-of-image rows are zero) and never in memory.
//
// Tiling (one workgroup = 4 waves, one wave per SIMD):
//   128 output channels x up to 448 output pixels (whole output rows of one
//   image); waves in a 2 x 2 grid, each 64 channels x 224 pixels = 2 x 7
//   v_mfma_f32_32x32x16_bf16 tiles, 224 accumulators per lane.
//   K loop: 16-channel stages, double-buffered in LDS:
//     weights  [tap 9][oc 128][ic 16] bf16, 32 B per (tap, oc), 36 KB per stage;
//              the two 16-byte halves are XOR-swizzled on bit 2 of oc so
//              16-byte reads of 8 consecutive rows hit distinct banks;
//     input    [row][col][ic 16] bf16 at 48 B per pixel (16 B pad) and a fixed
//              row pitch of ROWPX >= W + 2 pixels, <= 40 KB per stage.  The
//              odd 3 x 16 B pixel pitch makes reads of 8 consecutive pixels
//              conflict-free with no tap-dependent swizzle, so every B-operand
//              address is a per-lane base plus a compile-time tap offset.
//   Both are written transposed (ic contiguous per pixel / per channel) from
//   registers, since the MFMA operands need 8 consecutive k per lane while
//   NCHW and OIHW keep k strided.  Input stores are rotated by lane so that
//   8 neighbouring lanes write 8 different pixels of their 8-pixel groups.
//   A- and B-fragments are double-buffered in registers across the 9 taps.
// Epilogue: + bias[oc], fp32 stores straight into NCHW (coalesced along ow).
//
// Requirements (checked by the launcher): K = 3, stride 1, pad 1, C_in % 16
// == 0, C_in >= 32, C_out % 128 == 0, W % 8 == 0, 8 <= W <= 64, 16-byte aligned x and w.
// The kernel is instantiated for row pitches ROWPX = 10, 18, 34, 66 pixels.
#include "conv_internal.h"
#include "conv3x3_common.h"

namespace convfwd {
namespace {

constexpr int kThreads = 256;
constexpr int kOcTile = 128;
constexpr int kIcStage = 16;
constexpr int kWavePx = 224;                 // 7 MFMA columns of 32 pixels per wave
constexpr int kTilePx = 2 * kWavePx;         // 448 pixels per workgroup
constexpr int kNJ = kWavePx / 32;            // 7
constexpr int kWBufBytes = 9 * kOcTile * 32; // 36864
constexpr int kInBufBytes = 40960;
constexpr int kPixB = 48;                    // LDS bytes per input pixel (16 bf16 + pad)

// Tile plan.  Tiles are whole output rows [r0, r0 + R) of one image.  Each
// image is cut into chunks of `rows` rows; a chunk is split into `nparts` (1 to
// 3) tiles of part[0] >= part[1] >= part[2] rows.  With nparts == 1 the last
// chunk of an image may be short (the tile is clipped at H).  All first parts
// are dispatched, then all second parts, then all third parts; the kernel is
// persistent (workgroup b runs tiles b, b + G, b + 2G, ... for grid size G),
// so with G = number of chunks every workgroup runs one tile of each part,
// big ones first: the outputs of the early tiles stream out while the later
// ones compute, and only the small last tiles' stores remain at the end.
struct Plan {
    int part[3];
    int nparts;
    int rows;            // rows per chunk (sum of the parts)
    int chunks_per_img;
    int ntiles;          // total tiles = nparts * N * chunks_per_img
    int xcd_remap;       // 1: tiles that run at the same time on one XCD are neighbours
};

struct Tile { int n, r0, R; };

__host__ __device__ inline Tile decode_tile(const Plan &pl, int H, int b) {
    int t = b;
    const int per = pl.xcd_remap ? (pl.ntiles >> 3) : pl.ntiles;
    if (pl.xcd_remap) t = (b & 7) * per + (b >> 3);
    // within each range of `per` tiles: its chunks' first parts, then second, ...
    const int base = (t / per) * per, k = t - base, cpr = per / pl.nparts;
    const int part = k / cpr;
    const int chunk = base / pl.nparts + (k - part * cpr);
    Tile tl;
    tl.n = chunk / pl.chunks_per_img;
    const int c = chunk - tl.n * pl.chunks_per_img;
    int off = 0;
    for (int q = 0; q < part; ++q) off += pl.part[q];
    tl.r0 = c * pl.rows + off;
    tl.R = pl.part[part] < H - tl.r0 ? pl.part[part] : H - tl.r0;
    return tl;
}

// Where one thread loads the input of a tile from, and where it puts it in LDS.
struct LoadCtx {
    __amdgpu_buffer_rsrc_t xr;   // the tile's image
    uint32_t ivoff;              // byte offset of (ic group, row, 8-pixel group) at stage 0, or kOob
    uint32_t i_dst;              // LDS byte offset of the group's first pixel, channel half included
    bool in_active;
};

// Per-thread state shared by every tile of the workgroup.

struct KCtx {
    uint8_t *wbuf0, *ibuf0;
    lds_u8 *wlds0;               // wbuf0 as an LDS-space pointer (direct-to-LDS loads)
    __amdgpu_buffer_rsrc_t wr;   // this workgroup's 128 weight rows
    __amdgpu_buffer_rsrc_t wpr;  // packed weights of this workgroup's channel block
    uint32_t lane16;             // lane * 16
    int wave;                    // wave index (uniform)
    uint32_t w_voff;             // byte offset of (oc_l, ic group) at stage 0
    uint32_t w_dst;              // LDS byte offset of (tap 0, oc_l) with swizzle
    uint32_t stage_x_bytes;      // 16 channels of input: 16 * H * W * 2
    uint32_t chan_bytes;         // one channel plane: H * W * 2
};

__device__ __forceinline__ LoadCtx make_load_ctx(const uint16_t *x, int C, int H, int W, const Tile &tl,
                                                 int ROWPX) {
    LoadCtx l;
    const int64_t HW = (int64_t)H * W;
    l.xr = __builtin_amdgcn_make_buffer_rsrc((void *)(x + (int64_t)tl.n * C * HW), (short)0,
                                             (int)((int64_t)C * HW * 2), 0x00020000);
    // unit u -> (row rr, 8-pixel group pg, channel group g), rows fastest so
    // neighbouring lanes write LDS rows ROWPX pixels apart (at most 2-way conflicts)
    const int RR = tl.R + 2, pgs = W >> 3, tid = threadIdx.x;
    l.in_active = tid < 2 * RR * pgs;
    const int rr = tid % RR, rest = tid / RR;
    const int pg = rest % pgs, g = l.in_active ? rest / pgs : 0;
    const int ih = tl.r0 - 1 + rr;
    const bool valid = l.in_active && ih >= 0 && ih < H;
    l.ivoff = valid ? (uint32_t)(((int64_t)g * 8 * HW + (int64_t)ih * W + pg * 8) * 2) : kOob;
    l.i_dst = (uint32_t)((rr * ROWPX + pg * 8 + 1) * kPixB + g * 16);
    return l;
}

struct Stage { uint4 w[9]; uint4 in[8]; };

// Packed weights: stage s of this workgroup's weights is stored in global
// memory as the exact 36 KB LDS image, so it is copied by 9 direct-to-LDS
// loads per wave (1 KB contiguous each) with no registers or VALU work.
__device__ __forceinline__ void dma_w_stage(const KCtx &k, int s, int buf) {
#pragma unroll
    for (int q = 0; q < 9; ++q) {
        const int blk = k.wave * 9 + q;
        dma_1k(k.wlds0 + buf * kWBufBytes + blk * 1024, k.wpr, k.lane16, s * kWBufBytes + blk * 1024);
    }
}

// Transposed LDS writes of a loaded stage, in four parts so they can be spread
// between MFMAs: parts 0-1 weights (taps 0-4, 5-8), parts 2-3 input (pixels 0-3, 4-7).
template <int PART>
__device__ __forceinline__ void store_part(const KCtx &k, const LoadCtx &l, int buf, const Stage &st) {
    if (PART < 2) {
        // element e = icl*9 + tap of the 72 loaded -> [tap][oc][icl]
        const uint32_t *d = reinterpret_cast<const uint32_t *>(st.w);
        uint8_t *wb = k.wbuf0 + buf * kWBufBytes + k.w_dst;
#pragma unroll
        for (int t = PART * 5; t < (PART ? 9 : 5); ++t) {
            uint4 o;
            uint32_t *oo = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int e0 = (2 * m) * 9 + t, e1 = (2 * m + 1) * 9 + t;
                oo[m] = pack_halves(d[e0 >> 1], e0 & 1, d[e1 >> 1], e1 & 1);
            }
            *reinterpret_cast<uint4 *>(wb + t * (kOcTile * 32)) = o;
        }
    } else if (l.in_active) {
        // 8 channels x 8 pixels -> pixel j's 8 channels
        const uint32_t *v = reinterpret_cast<const uint32_t *>(st.in);   // v[e*4 + j/2]
        uint8_t *ib = k.ibuf0 + buf * kInBufBytes + l.i_dst;
#pragma unroll
        for (int j = (PART - 2) * 4; j < (PART - 2) * 4 + 4; ++j) {
            const int dj = j >> 1, h = j & 1;
            uint4 o;
            o.x = pack_halves(v[0 * 4 + dj], h, v[1 * 4 + dj], h);
            o.y = pack_halves(v[2 * 4 + dj], h, v[3 * 4 + dj], h);
            o.z = pack_halves(v[4 * 4 + dj], h, v[5 * 4 + dj], h);
            o.w = pack_halves(v[6 * 4 + dj], h, v[7 * 4 + dj], h);
            *reinterpret_cast<uint4 *>(ib + j * kPixB) = o;
        }
    }
}

// Split issue: weights and input loads of one stage separately, so each can
// go out as soon as the registers it overwrites have been consumed.
__device__ __forceinline__ void issue_w_loads(const KCtx &k, int s, Stage &st) {
    const uint32_t ws = (uint32_t)s * (kIcStage * 9 * 2);
#pragma unroll
    for (int q = 0; q < 9; ++q) st.w[q] = bload16(k.wr, k.w_voff + q * 16, ws);
}
__device__ __forceinline__ void issue_x_loads(const KCtx &k, const LoadCtx &l, int s, Stage &st) {
    const uint32_t xs = (uint32_t)s * k.stage_x_bytes;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.in[e] = bload16(l.xr, l.ivoff, xs + e * k.chan_bytes);
}

// Column count a wave actually runs for nj pixel columns: one of the
// instantiated 7, 6, 4, 2 (extra columns compute on padding and are not stored).
__host__ __device__ constexpr int nj_variant(int nj) { return nj >= 7 ? 7 : nj >= 5 ? 6 : nj >= 3 ? 4 : 2; }

// One tile for a wave that runs NJ pixel columns (ROWPX: LDS row pitch of the
// input tile).  On entry LDS buffer `buf` holds stage 0 of this tile.  While
// stage s is multiplied out of `buf`, registers `st` hold stage s+1, which is
// written transposed into buf ^ 1 between the MFMAs of taps 5-8; right after
// each part is written, the loads of stage s+2 go out into the freed
// registers, so every load has about eight taps of MFMA work to arrive.
// Within a tap, the next tap's A fragments are read first; B fragments live in
// one rotating set (column j's fragment is re-read for the next tap right
// after its two MFMAs).  After the last stage, the next tile's stage 0 is
// loaded while this tile's outputs are stored, then written to LDS, so on
// exit `buf` holds the next tile's stage 0.  Requires S >= 2.
template <int NJ, int ROWPX, bool PACKED>
__device__ __forceinline__ void tile_body(const KCtx &k, const LoadCtx &lc, const LoadCtx &lcn,
                                          bool has_next, int S, int &buf, uint32_t a_off,
                                          const uint32_t (&b_off)[kNJ], __amdgpu_buffer_rsrc_t br,
                                          uint32_t bvoff, int lane,
                                          int wm, int pbeg, int pend, __amdgpu_buffer_rsrc_t yr,
                                          uint32_t half_rows, uint32_t row_bytes) {
    // Accumulator tile (i, j) is D = X_tile (32 pixels x 16 k) * W_tile (16 k x
    // 32 channels): lane l holds channel l%32 and pixels 8*(r/4) + 4*(l/32) +
    // r%4 in slot r, so slots 4k..4k+3 are four consecutive output pixels of
    // one channel.  Accumulators start from that channel's bias (a buffer
    // with no records when there is no bias: the loads return 0).
    f32x16_t acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float bv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(br, (int)(bvoff + i * 32 * 4), 0, 0));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = bv;
    }
    Stage st;
    if (!PACKED) issue_w_loads(k, 1, st);
    issue_x_loads(k, lc, 1, st);
    for (int s = 0; s < S; ++s) {
        const bool st_ok = s + 1 < S;          // registers hold stage s+1
        const bool ld_ok = s + 2 < S;          // stage s+2 to load
        // packed weights of stage s+1 go straight to buf ^ 1 (free since the
        // barrier that ended stage s-1) and must land before this stage's barrier
        if (PACKED && st_ok) dma_w_stage(k, s + 1, buf ^ 1);
        const uint8_t *wb = k.wbuf0 + buf * kWBufBytes + a_off;
        const uint8_t *ib = k.ibuf0 + buf * kInBufBytes;
        uint4 a[2][2], b[NJ];
        auto fetch_a = [&](int t, int set) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[set][i] = *reinterpret_cast<const uint4 *>(wb + t * (kOcTile * 32) + i * 32 * 32);
        };
        auto fetch_b = [&](int t, int j) {
            const int toff = ((t / 3) * ROWPX + (t % 3)) * kPixB;     // compile-time per tap
            b[j] = *reinterpret_cast<const uint4 *>(ib + b_off[j] + toff);
        };
        fetch_a(0, 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) fetch_b(0, j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            if (t + 1 < 9) fetch_a(t + 1, (t + 1) & 1);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[i][j] = mfma32x32x16(b[j], a[t & 1][i], acc[i][j]);
                if (t + 1 < 9) fetch_b(t + 1, j);
            }
            if (st_ok) {
                if (!PACKED && t == 5) store_part<0>(k, lc, buf ^ 1, st);
                if (!PACKED && t == 6) {
                    store_part<1>(k, lc, buf ^ 1, st);
                    if (ld_ok) issue_w_loads(k, s + 2, st);
                }
                if (t == 7) store_part<2>(k, lc, buf ^ 1, st);
                if (t == 8) {
                    store_part<3>(k, lc, buf ^ 1, st);
                    if (ld_ok) issue_x_loads(k, lc, s + 2, st);
                }
            }
            // Pin the order within a tap: the two A reads for tap t+1, then for
            // each column its two MFMAs followed by its B read for tap t+1.
            // Nothing moves across the tap boundary.
            if (t + 1 < 9) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * NJ, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (PACKED) {
            // the weight copy into buf ^ 1 was issued before the 8 input loads
            // of stage s+2 (vector-memory counters complete in order)
            if (ld_ok) CONV3X3_WAIT_VMCNT(8);
            else CONV3X3_WAIT_VMCNT(0);
        }
        __syncthreads();
        buf ^= 1;
    }

    // ---- next tile's stage 0 in flight while this tile's outputs are stored
    if (has_next) {
        if (PACKED) dma_w_stage(k, 0, buf);
        else issue_w_loads(k, 0, st);
        issue_x_loads(k, lcn, 0, st);
    }
    // y[n][oc][r0 + p/W][p%W] = acc: one 16-byte store per 4 consecutive
    // pixels (56 stores per wave for 7 columns, few enough to stay in flight
    // while the next tile computes).  Channel row offset in soffset, pixel
    // offset in the immediate; groups past the tile (always whole, since the
    // tile's pixel count is a multiple of 8) get an out-of-range offset and
    // their stores are dropped.
    const int half = (lane >> 5) & 1;
    const uint32_t ylane = (uint32_t)(lane & 31) * row_bytes + (uint32_t)(pbeg + 4 * half) * 4;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool ok = pbeg + j * 32 + q * 8 + 4 * half < pend;
            const uint32_t vo = ok ? ylane : kOob;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const u32x4_t v = {__float_as_uint(acc[i][j][4 * q]), __float_as_uint(acc[i][j][4 * q + 1]),
                                   __float_as_uint(acc[i][j][4 * q + 2]), __float_as_uint(acc[i][j][4 * q + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(v, yr, (int)(vo + (uint32_t)(j * 32 + q * 8) * 4),
                                                       (int)((uint32_t)(wm * 64 + i * 32) * row_bytes), 0);
            }
        }
    if (has_next) {
        if (!PACKED) {
            store_part<0>(k, lcn, buf, st);
            store_part<1>(k, lcn, buf, st);
        }
        store_part<2>(k, lcn, buf, st);
        store_part<3>(k, lcn, buf, st);
    }
    if (PACKED) CONV3X3_WAIT_VMCNT(0);
    __syncthreads();
}

// The kernel: a persistent loop over this workgroup's tiles.  PACKED: `wp`
// holds the weights repacked by pack_w3x3_kernel (per channel block and
// stage, the LDS image), loaded without transposes; otherwise `w` (OIHW) is
// transposed on the way into LDS.
template <int ROWPX, bool PACKED>
__global__ __launch_bounds__(kThreads, 1)
void conv3x3s1_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                      const uint16_t *__restrict__ wp, const float *__restrict__ bias,
                      float *__restrict__ y, int C, int H, int W, int Co, Plan plan) {
    __shared__ __align__(16) uint8_t smem[2 * kWBufBytes + 2 * kInBufBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int wm = wave >> 1, wn = wave & 1;
    const int ocb = blockIdx.y * kOcTile;
    const int64_t HW = (int64_t)H * W;
    const int half = lane >> 5, l32 = lane & 31;

    KCtx k;
    k.wbuf0 = smem;
    k.ibuf0 = smem + 2 * kWBufBytes;
    k.wlds0 = (lds_u8 *)smem;
    k.wave = wave;
    k.lane16 = (uint32_t)lane * 16;
    if (PACKED)
        k.wpr = __builtin_amdgcn_make_buffer_rsrc((void *)(wp + (int64_t)ocb * C * 9), (short)0,
                                                  kOcTile * C * 9 * 2, 0x00020000);
    k.wr = __builtin_amdgcn_make_buffer_rsrc((void *)(w + (int64_t)ocb * C * 9), (short)0,
                                             kOcTile * C * 9 * 2, 0x00020000);
    const int w_ocl = tid & (kOcTile - 1), w_g = tid >> 7;
    k.w_voff = (uint32_t)((w_ocl * C + w_g * 8) * 9 * 2);
    k.w_dst = (uint32_t)(w_ocl * 32 + ((w_g ^ wswz(w_ocl)) * 16));
    k.chan_bytes = (uint32_t)(HW * 2);
    k.stage_x_bytes = (uint32_t)(HW * 2 * kIcStage);
    const uint32_t a_off = (uint32_t)((wm * 64 + l32) * 32 + ((half ^ wswz(l32)) * 16));
    // bias rows of this wave: 64 channels from ocb + wm*64; lane half adds 4 rows
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(bias ? bias + ocb + wm * 64 : y), (short)0, bias ? 64 * 4 : 0, 0x00020000);
    const uint32_t bvoff = (uint32_t)l32 * 4;
    const uint32_t row_bytes = (uint32_t)(HW * 4);
    const uint32_t half_rows = (uint32_t)half * 4 * row_bytes;

    // Zero both input buffers once: the edge columns (0 and W+1) are never
    // written again and stay zero for every stage (left/right padding).
    for (int i = tid; i < 2 * kInBufBytes / 16; i += kThreads)
        reinterpret_cast<uint4 *>(k.ibuf0)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();

    const int S = C / kIcStage;
    const int G = gridDim.x;
    int f = blockIdx.x;
    Tile cur = decode_tile(plan, H, f);
    LoadCtx lc = make_load_ctx(x, C, H, W, cur, ROWPX);
    {   // prologue: stage 0 of the first tile into LDS buffer 0
        Stage st;
        if (PACKED) dma_w_stage(k, 0, 0);
        else issue_w_loads(k, 0, st);
        issue_x_loads(k, lc, 0, st);
        if (!PACKED) {
            store_part<0>(k, lc, 0, st);
            store_part<1>(k, lc, 0, st);
        }
        store_part<2>(k, lc, 0, st);
        store_part<3>(k, lc, 0, st);
        if (PACKED) CONV3X3_WAIT_VMCNT(0);
        __syncthreads();
    }
    int buf = 0;
    for (;;) {
        const int fn = f + G;
        const bool has_next = fn < plan.ntiles;
        const Tile nxt = has_next ? decode_tile(plan, H, fn) : cur;
        const LoadCtx lcn = make_load_ctx(x, C, H, W, nxt, ROWPX);

        // this wave's pixel range: the tile's npx pixels split at a multiple of
        // 32 so both pixel-waves run about the same number of MFMA columns
        const int npx = cur.R * W;
        const int wsplit = ((npx + 63) / 64) * 32;
        const int pbeg = wn ? wsplit : 0;
        const int pend = wn ? npx : min(npx, wsplit);
        const int nj = __builtin_amdgcn_readfirstlane((pend - pbeg + 31) >> 5);   // 0..7
        // B columns: tile pixel p -> LDS pixel (p/W)*ROWPX + p%W (tap (0,0)), channel half at +16 B
        uint32_t b_off[kNJ];
#pragma unroll
        for (int j = 0; j < kNJ; ++j) {
            const int p = pbeg + j * 32 + l32;
            const int pr = p / W;
            b_off[j] = (uint32_t)((pr * ROWPX + (p - pr * W)) * kPixB + half * 16);
        }
        const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(y + ((int64_t)cur.n * Co + ocb) * HW + (int64_t)cur.r0 * W), (short)0,
            (int)((int64_t)kOcTile * HW * 4 - (int64_t)cur.r0 * W * 4), 0x00020000);

#define CONV3X3_TILE(NJV)                                                                       \
    tile_body<NJV, ROWPX, PACKED>(k, lc, lcn, has_next, S, buf, a_off, b_off, br, bvoff, lane, wm, pbeg, \
                          pend, yr, half_rows, row_bytes)
        switch (nj_variant(nj)) {
            case 7: CONV3X3_TILE(7); break;
            case 6: CONV3X3_TILE(6); break;
            case 4: CONV3X3_TILE(4); break;
            default: CONV3X3_TILE(2); break;
        }
#undef CONV3X3_TILE
        if (!has_next) break;
        f = fn;
        cur = nxt;
        lc = lcn;
    }
}

// Repack OIHW 3x3 weights for the PACKED kernel: for every 128-channel block
// and 16-channel stage, the 36 KB image that stage occupies in LDS
// ([tap 9][oc 128][ic 16], 16-byte halves swizzled as in wswz).  One thread
// per 16-byte unit of the packed array, in the array's order (so the stores
// of a wave are 1 KB contiguous): it gathers the unit's 8 input channels of
// one tap straight from the OIHW weights, a single memory round trip.
__global__ __launch_bounds__(256)
void pack_w3x3_kernel(const uint16_t *__restrict__ w, uint16_t *__restrict__ wp, int C, int Co) {
    const int S = C / kIcStage;
    const int64_t total = (int64_t)Co * S * 18;
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= total) return;
    // u = (((ocb * S + st) * 9 + t) * kOcTile + ocl) * 2 + slot
    const int slot = (int)(u & 1);
    int64_t r = u >> 1;
    const int ocl = (int)(r % kOcTile);
    r /= kOcTile;
    const int t = (int)(r % 9);
    r /= 9;
    const int st = (int)(r % S), ocb = (int)(r / S);
    const int h = slot ^ wswz(ocl);
    const uint16_t *src = w + ((int64_t)(ocb * kOcTile + ocl) * C + st * kIcStage + h * 8) * 9 + t;
    uint16_t e8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) e8[e] = src[e * 9];
    reinterpret_cast<uint4 *>(wp)[u] = pack8(e8);
}

// MFMA column steps (32 pixels each) that the busier pixel-wave of a tile runs.
int tile_steps(int npx) {
    const int wsplit = ((npx + 63) / 64) * 32;
    const int nj0 = (wsplit < npx ? wsplit : npx + 31) / 32, nj1 = (npx - wsplit + 31) / 32;
    const int v0 = nj_variant(nj0 > 0 ? nj0 : 0), v1 = nj_variant(nj1 > 0 ? nj1 : 0);
    return v0 > v1 ? v0 : v1;
}

// LDS row pitch (pixels) of the input tile for a width W: the smallest
// instantiated pitch that holds W + 2 columns.
int row_px_for(int W) { return W <= 8 ? 10 : W <= 16 ? 18 : W <= 32 ? 34 : 66; }

// One past the largest LDS input-buffer byte a tile of R rows can touch:
// pixel columns run up to 31 pixels past the tile, plus the kh = 2 row offset
// and the kw = 2 column offset; each read is 16 bytes at +0 or +16.
int tile_lds_bytes(int R, int W) {
    const int rowpx = row_px_for(W);
    const int npx = R * W, wsplit = ((npx + 63) / 64) * 32;
    const int nj1 = (npx - wsplit + 31) / 32;
    const int nj0 = (npx < wsplit ? npx : wsplit) / 32 + ((npx < wsplit && npx % 32) ? 1 : 0);
    const int pmax0 = nj_variant(nj0) * 32 - 1;
    const int pmax1 = wsplit + nj_variant(nj1 > 0 ? nj1 : 0) * 32 - 1;
    const int pmax = pmax0 > pmax1 ? pmax0 : pmax1;
    const int q = (pmax / W + 2) * rowpx + (W - 1) + 2;
    const int q_store = (R + 1) * rowpx + W;
    return (q > q_store ? q : q_store) * kPixB + 32;
}

// Estimated time of a plan on the persistent grid (workgroup b runs tiles b,
// b + G, ...; one workgroup per CU, all resident).  Unit: one MFMA column step
// over all K stages as the kernel runs it (about twice the bare MFMA time).
//  - a tile costs its busier pixel-wave's column steps, but no less than a
//    floor: every stage also moves a whole 36 KB weight image into LDS and
//    passes two barriers, whatever the tile's width;
//  - a tile that is not its workgroup's last ends with a stall: the vector
//    memory counter retires in order, so the first wait on a load issued
//    after the tile's output stores also waits for those stores, and all
//    workgroups reach that point together (chip-wide burst at ~6 TB/s);
//  - the outputs of the last tiles drain after compute ends.
int grid_size(const Plan &pl, int slots) { return pl.ntiles < slots ? pl.ntiles : slots; }

double plan_cost(const Shape &sh, const Plan &pl, int slots) {
    constexpr double kMinTileSteps = 4.0, kTileOverhead = 0.3, kDrainBps = 6.0e12;
    const int G = grid_size(pl, slots);
    const int ncb = sh.Co / kOcTile;
    const double unit_s = 2.0 * 18.0 * (sh.C / kIcStage) * 32.0 / 2.0e9;   // 18*S MFMAs, 32 clk at ~2 GHz, x2
    const double burst = (double)kOcTile * 4.0 * G * ncb / kDrainBps / unit_s;  // per output pixel of a tile
    double worst = 0, last_px = 0;
    for (int b = 0; b < G; ++b) {
        double load = 0;
        int lastR = 0;
        for (int f = b; f < pl.ntiles; f += G) {
            const Tile tl = decode_tile(pl, sh.H, f);
            const double st = tile_steps(tl.R * sh.W);
            load += (st > kMinTileSteps ? st : kMinTileSteps) + kTileOverhead;
            if (f + G < pl.ntiles) load += burst * tl.R * sh.W;
            lastR = tl.R;
        }
        if (load > worst) worst = load;
        last_px += (double)lastR * sh.W;
    }
    return worst + last_px * kOcTile * 4.0 * ncb / kDrainBps / unit_s;
}

void set_remap(Plan &p) {
    p.xcd_remap = (p.ntiles % 8 == 0 && (p.ntiles / 8) % p.nparts == 0) ? 1 : 0;
}

// Resident workgroups per output-channel block: one per CU in total.
int slots_for(const Shape &sh, int num_cu) {
    const int ncb = sh.Co / kOcTile;
    return num_cu / ncb > 0 ? num_cu / ncb : 1;
}

// Choose the row tiling among uniform tiles of R rows and chunks of two or
// three decreasing parts that divide each image's rows, by the smallest
// estimated time.
Plan make_plan(const Shape &sh, int slots) {
    const int W = sh.W, H = sh.H, N = sh.N;
    int rmax = kTilePx / W;
    while (rmax > 1 && tile_lds_bytes(rmax, W) > kInBufBytes) --rmax;
    Plan best{};
    double best_cost = 1e300;
    auto consider = [&](int r0, int r1, int r2) {
        Plan p{};
        p.part[0] = r0; p.part[1] = r1; p.part[2] = r2;
        p.nparts = 1 + (r1 > 0) + (r2 > 0);
        p.rows = r0 + r1 + r2;
        if (p.nparts == 1) {
            p.chunks_per_img = (H + r0 - 1) / r0;
        } else {
            if (H % p.rows) return;
            p.chunks_per_img = H / p.rows;
        }
        p.ntiles = p.nparts * N * p.chunks_per_img;
        set_remap(p);
        const double c = plan_cost(sh, p, slots);
        if (c < best_cost * 0.999) { best_cost = c; best = p; }
    };
    for (int a = 1; a <= rmax && a <= H; ++a) {
        if (tile_lds_bytes(a, W) > kInBufBytes) continue;
        consider(a, 0, 0);
        for (int b = 1; b <= a; ++b) {
            consider(a, b, 0);
            for (int c = 1; c <= b; ++c) consider(a, b, c);
        }
    }
    return best;
}

}  // namespace

void launch_pack_w3x3(const Shape &sh, const uint16_t *w, uint16_t *wpack, hipStream_t st) {
    // a grouped layer packs as a layer of C_in / groups input channels
    const int64_t units = (int64_t)sh.Co * (sh.Cg() / kIcStage) * 18;
    hipLaunchKernelGGL(pack_w3x3_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st, w, wpack, sh.Cg(),
                       sh.Co);
}

bool conv3x3s1_supported(const Shape &sh, const void *x, const void *w) {
    const int64_t HW = (int64_t)sh.H * sh.W;
    return sh.plain() && sh.plain_io() && sh.ndim == 2 && sh.K == 3 && sh.s == 1 && sh.p == 1 && sh.C % kIcStage == 0 &&
           sh.C >= 2 * kIcStage &&
           sh.Co % kOcTile == 0 && sh.W % 8 == 0 && sh.W >= 8 && sh.W <= 64 &&
           (int64_t)sh.C * HW * 2 < (INT64_C(1) << 31) &&            // one image within a buffer range
           (int64_t)kOcTile * HW * 4 < (INT64_C(1) << 31) &&         // one output block within a buffer range
           (int64_t)kOcTile * sh.C * 9 * 2 < (INT64_C(1) << 31) &&
           ((uintptr_t)x % 16) == 0 && ((uintptr_t)w % 16) == 0 && tile_lds_bytes(1, sh.W) <= kInBufBytes;
}

size_t conv3x3s1_workspace_bytes(const Shape &sh) {
    return (size_t)sh.Co * sh.Cg() * 9 * 2;          // packed weights (C_in / groups per output channel)
}

hipError_t launch_conv3x3s1_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, uint16_t *wpack,
                                 const float *bias, float *y, hipStream_t st, bool prepacked) {
    // CU count of the current device and the last plan, per host thread (the
    // plan depends only on (N, H, W) and the CU count).
    thread_local int cached_dev = -1, num_cu = 256;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorNoDevice;
    if (dev != cached_dev) {
        int n = 0;
        num_cu = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
                     ? n : 256;
        cached_dev = dev;
    }
    thread_local int last_n = -1, last_h = -1, last_w = -1, last_cu = -1;
    thread_local Plan last{};
    if (sh.N != last_n || sh.H != last_h || sh.W != last_w || num_cu != last_cu) {
        last = make_plan(sh, slots_for(sh, num_cu));
        last_n = sh.N; last_h = sh.H; last_w = sh.W; last_cu = num_cu;
    }
    const Plan pl = last;
    if (wpack && !prepacked) launch_pack_w3x3(sh, w, wpack, st);
    dim3 grid((unsigned)grid_size(pl, slots_for(sh, num_cu)), (unsigned)(sh.Co / kOcTile));
#define CONV3X3_LAUNCH(RP)                                                                          \
    do {                                                                                            \
        if (wpack)                                                                                  \
            hipLaunchKernelGGL((conv3x3s1_kernel<RP, true>), grid, dim3(kThreads), 0, st, x, w, wpack, \
                               bias, y, sh.C, sh.H, sh.W, sh.Co, pl);                               \
        else                                                                                        \
            hipLaunchKernelGGL((conv3x3s1_kernel<RP, false>), grid, dim3(kThreads), 0, st, x, w, w,   \
                               bias, y, sh.C, sh.H, sh.W, sh.Co, pl);                               \
    } while (0)
    switch (row_px_for(sh.W)) {
        case 10: CONV3X3_LAUNCH(10); break;
        case 18: CONV3X3_LAUNCH(18); break;
        case 34: CONV3X3_LAUNCH(34); break;
        default: CONV3X3_LAUNCH(66); break;
    }
#undef CONV3X3_LAUNCH
    return hipGetLastError();
}

}  // namespace convfwd
