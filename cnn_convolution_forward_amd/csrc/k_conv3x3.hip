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
// == 0, C_out % 128 == 0, W % 8 == 0, 8 <= W <= 64, 16-byte aligned x and w.
// The kernel is instantiated for row pitches ROWPX = 10, 18, 34, 66 pixels.
#include "conv_internal.h"
#include "mfma_common.h"

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

// Tile plan.  Tiles are whole output rows [r0, r0 + R) of one image.  With
// Rb == 0 each image is cut into ceil(H/Ra) tiles (the last may be short).
// With Rb > 0 each image is cut into chunks of Ra + Rb rows; every chunk gives
// one tile of its first Ra rows (group A) and one of its last Rb rows (group
// B).  The kernel is persistent: workgroup b runs tiles b, b + G, b + 2G, ...
// (G = grid size), so with G = number of chunks each workgroup runs one A and
// one B tile.
struct Plan {
    int Ra, Rb;
    int tiles_per_img;   // tiles (Rb == 0) or chunks (Rb > 0) per image
    int ntiles;          // total tiles
    int xcd_remap;       // 1: tiles that run at the same time on one XCD are neighbours
};

struct Tile { int n, r0, R; };

__device__ __forceinline__ Tile decode_tile(const Plan &pl, int H, int b) {
    int t = b;
    if (pl.xcd_remap) {
        const int per = pl.ntiles >> 3;
        t = (b & 7) * per + (b >> 3);
    }
    Tile tl;
    if (pl.Rb == 0) {
        tl.n = t / pl.tiles_per_img;
        tl.r0 = (t - tl.n * pl.tiles_per_img) * pl.Ra;
        tl.R = min(pl.Ra, H - tl.r0);
    } else {
        // within each XCD's contiguous range: first its A tiles, then its B tiles
        const int per = pl.xcd_remap ? (pl.ntiles >> 3) : pl.ntiles;
        const int base = (t / per) * per, k = t - base, half = per >> 1;
        const int chunk = (base >> 1) + (k < half ? k : k - half);
        tl.n = chunk / pl.tiles_per_img;
        const int c = chunk - tl.n * pl.tiles_per_img;
        tl.r0 = c * (pl.Ra + pl.Rb) + (k < half ? 0 : pl.Ra);
        tl.R = k < half ? pl.Ra : pl.Rb;
    }
    return tl;
}

// 16-byte halves of a 32-byte weight row are swapped on bit 2 xor bit 3 of the
// row, so 16-byte accesses of 8 (32 banks) or 16 (64 banks) consecutive rows
// reach distinct banks.
__device__ __forceinline__ int wswz(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

// lo 16 bits from half `ha` of a, hi 16 bits from half `hb` of b (one v_perm_b32).
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, int ha, uint32_t b, int hb) {
    const uint32_t sel = (uint32_t)(2 * ha) | ((uint32_t)(2 * ha + 1) << 8) |
                         ((uint32_t)(4 + 2 * hb) << 16) | ((uint32_t)(5 + 2 * hb) << 24);
    return __builtin_amdgcn_perm(b, a, sel);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr uint32_t kOob = 0x80000000u;     // buffer offset past any valid byte: loads 0, stores dropped

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
    __amdgpu_buffer_rsrc_t wr;   // this workgroup's 128 weight rows
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

// Issue the global (buffer) loads of stage s.
__device__ __forceinline__ void issue_loads(const KCtx &k, const LoadCtx &l, int s, Stage &st) {
    const uint32_t ws = (uint32_t)s * (kIcStage * 9 * 2);
#pragma unroll
    for (int q = 0; q < 9; ++q) st.w[q] = bload16(k.wr, k.w_voff + q * 16, ws);
    const uint32_t xs = (uint32_t)s * k.stage_x_bytes;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.in[e] = bload16(l.xr, l.ivoff, xs + e * k.chan_bytes);
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

// All K stages of one tile for a wave that owns NJ pixel columns (ROWPX: the
// LDS row pitch of the input tile).  Stage s computes from LDS buffer `buf`
// while the loads of the next stage -- stage s+1 of this tile, or stage 0 of
// the next tile -- are in flight and then written, transposed, into buf ^ 1
// between the MFMAs of taps 4-7.
template <int NJ, int ROWPX>
__device__ __forceinline__ void run_tile(const KCtx &k, const LoadCtx &lcur, const LoadCtx &lnext,
                                         bool has_next, int S, int &buf, const uint32_t (&b_off)[kNJ],
                                         uint32_t a_off, const float *bias_rows, int lane,
                                         __amdgpu_buffer_rsrc_t yr, uint32_t ylane, uint32_t half_rows,
                                         uint32_t row_bytes, int wm, int pbeg, int pend) {
    constexpr int NB = NJ > 0 ? NJ : 1;
    // accumulators start from the bias of their output channel
    f32x16_t acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float bv = bias_rows ? bias_rows[i * 32 + mfma32_row(r, lane)] : 0.f;
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j][r] = bv;
        }
    for (int s = 0; s < S; ++s) {
        const bool pf = (s + 1 < S) || has_next;
        const LoadCtx &lp = (s + 1 < S) ? lcur : lnext;
        const int ps = (s + 1 < S) ? s + 1 : 0;
        Stage st;
        if (pf) issue_loads(k, lp, ps, st);
        const uint8_t *wb = k.wbuf0 + buf * kWBufBytes + a_off;
        const uint8_t *ib[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) ib[j] = k.ibuf0 + buf * kInBufBytes + b_off[j];
        uint4 a[2][2], b[2][NB];
        auto fetch = [&](int t, int set) {
            const int toff = ((t / 3) * ROWPX + (t % 3)) * kPixB;     // compile-time per tap
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[set][i] = *reinterpret_cast<const uint4 *>(wb + t * (kOcTile * 32) + i * 32 * 32);
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[set][j] = *reinterpret_cast<const uint4 *>(ib[j] + toff);
        };
        fetch(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            if (t + 1 < 9) fetch(t + 1, (t + 1) & 1);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[i][j] = mfma32x32x16(a[t & 1][i], b[t & 1][j], acc[i][j]);
            if (pf) {
                if (t == 4) store_part<0>(k, lp, buf ^ 1, st);
                if (t == 5) store_part<1>(k, lp, buf ^ 1, st);
                if (t == 6) store_part<2>(k, lp, buf ^ 1, st);
                if (t == 7) store_part<3>(k, lp, buf ^ 1, st);
            }
            // Within a tap: the next tap's operand reads first, then this tap's
            // MFMAs (whose operands arrived during the previous tap).  Nothing
            // moves across the tap boundary.
            if (t + 1 < 9) __builtin_amdgcn_sched_group_barrier(0x100, 2 + NJ, 0);   // DS reads
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * NJ, 0);                  // MFMAs
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        buf ^= 1;
    }
    // ---- epilogue: y[n][oc][r0 + p/W][p%W] = acc.  Buffer stores with the
    // row offset in soffset and the column in the immediate; lanes past the
    // tile get an out-of-range offset and their stores are dropped.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bool ok = pbeg + j * 32 + (lane & 31) < pend;
        const uint32_t vo = ok ? ylane + j * 128 + half_rows : kOob;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t row = (uint32_t)(wm * 64 + i * 32 + 8 * (r >> 2) + (r & 3));   // + 4*half via voffset
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), yr, (int)vo,
                                                      (int)(row * row_bytes), 0);
            }
    }
}

template <int ROWPX>
__global__ __launch_bounds__(kThreads, 1)
void conv3x3s1_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                      const float *__restrict__ bias, float *__restrict__ y,
                      int C, int H, int W, int Co, Plan plan) {
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
    k.wr = __builtin_amdgcn_make_buffer_rsrc((void *)(w + (int64_t)ocb * C * 9), (short)0,
                                             kOcTile * C * 9 * 2, 0x00020000);
    const int w_ocl = tid & (kOcTile - 1), w_g = tid >> 7;
    k.w_voff = (uint32_t)((w_ocl * C + w_g * 8) * 9 * 2);
    k.w_dst = (uint32_t)(w_ocl * 32 + ((w_g ^ wswz(w_ocl)) * 16));
    k.chan_bytes = (uint32_t)(HW * 2);
    k.stage_x_bytes = (uint32_t)(HW * 2 * kIcStage);
    const uint32_t a_off = (uint32_t)((wm * 64 + l32) * 32 + ((half ^ wswz(l32)) * 16));

    const float *bias_rows = bias ? bias + ocb + wm * 64 : nullptr;

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
    {   // prologue: stage 0 of the first tile
        Stage st;
        issue_loads(k, lc, 0, st);
        store_part<0>(k, lc, 0, st);
        store_part<1>(k, lc, 0, st);
        store_part<2>(k, lc, 0, st);
        store_part<3>(k, lc, 0, st);
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
        const uint32_t ylane = (uint32_t)((pbeg + l32) * 4);
        const uint32_t row_bytes = (uint32_t)(HW * 4);
        const uint32_t half_rows = (uint32_t)half * 4 * row_bytes;

#define CONV3X3_RUN(NJV)                                                                        \
    run_tile<NJV, ROWPX>(k, lc, lcn, has_next, S, buf, b_off, a_off, bias_rows, lane, yr, ylane, \
                         half_rows, row_bytes, wm, pbeg, pend)
        switch (nj) {
            case 7: CONV3X3_RUN(7); break;
            case 6: CONV3X3_RUN(6); break;
            case 5: CONV3X3_RUN(5); break;
            case 4: CONV3X3_RUN(4); break;
            case 3: CONV3X3_RUN(3); break;
            case 2: CONV3X3_RUN(2); break;
            case 1: CONV3X3_RUN(1); break;
            default: CONV3X3_RUN(0); break;
        }
#undef CONV3X3_RUN
        if (!has_next) break;
        f = fn;
        cur = nxt;
        lc = lcn;
    }
}

// MFMA column steps (32 pixels each) of a tile's busier pixel-wave.
int tile_steps(int npx) { return (npx + 63) / 64; }

// LDS row pitch (pixels) of the input tile for a width W: the smallest
// instantiated pitch that holds W + 2 columns.
int row_px_for(int W) { return W <= 8 ? 10 : W <= 16 ? 18 : W <= 32 ? 34 : 66; }

// One past the largest LDS input-buffer byte a tile of R rows can touch:
// pixel columns run up to 31 pixels past the tile, plus the kh = 2 row offset
// and the kw = 2 column offset; each read is 16 bytes at +0 or +16.
int tile_lds_bytes(int R, int W) {
    const int rowpx = row_px_for(W);
    const int npx = R * W, wsplit = ((npx + 63) / 64) * 32;
    const int pmax = wsplit + ((npx - wsplit + 31) / 32) * 32 - 1;
    const int q = (pmax / W + 2) * rowpx + (W - 1) + 2;
    const int q_store = (R + 1) * rowpx + W;
    return (q > q_store ? q : q_store) * kPixB + 32;
}

// Makespan of a plan on the persistent grid: workgroup b runs tiles b, b + G,
// ... (G = grid size, one workgroup per CU, all resident at once); a tile
// costs its MFMA column steps plus a fixed overhead for the pipeline fill and
// the output stores.
int grid_size(const Plan &pl, int slots) { return pl.ntiles < slots ? pl.ntiles : slots; }

double makespan(const Shape &sh, const Plan &pl, int slots) {
    const int G = grid_size(pl, slots);
    double worst = 0;
    for (int b = 0; b < G; ++b) {
        double load = 0;
        for (int f = b; f < pl.ntiles; f += G) {
            int t = f;
            if (pl.xcd_remap) t = (f & 7) * (pl.ntiles >> 3) + (f >> 3);
            int R;
            if (pl.Rb == 0) {
                const int r0 = (t % pl.tiles_per_img) * pl.Ra;
                R = pl.Ra < sh.H - r0 ? pl.Ra : sh.H - r0;
            } else {
                const int per = pl.xcd_remap ? (pl.ntiles >> 3) : pl.ntiles;
                R = (t % per) < (per >> 1) ? pl.Ra : pl.Rb;
            }
            load += tile_steps(R * sh.W) + 0.3;
        }
        if (load > worst) worst = load;
    }
    return worst;
}

void set_remap(Plan &p) {
    p.xcd_remap = (p.ntiles % 8 == 0 && (p.Rb == 0 || (p.ntiles / 8) % 2 == 0)) ? 1 : 0;
}

// Choose the row tiling among uniform tiles of R rows and (Ra, Rb) chunk pairs
// that divide each image's rows, by the smallest simulated makespan.
// Resident workgroups per output-channel block: one per CU in total.
int slots_for(const Shape &sh, int num_cu) {
    const int ncb = sh.Co / kOcTile;
    return num_cu / ncb > 0 ? num_cu / ncb : 1;
}

Plan make_plan(const Shape &sh, int num_cu) {
    const int W = sh.W, H = sh.H, N = sh.N;
    int rmax = kTilePx / W;
    while (rmax > 1 && tile_lds_bytes(rmax, W) > kInBufBytes) --rmax;
    Plan best{};
    double best_cost = 1e300;
    for (int R = 1; R <= rmax && R <= H; ++R) {
        if (tile_lds_bytes(R, W) > kInBufBytes) continue;
        Plan p{R, 0, (H + R - 1) / R, 0, 0};
        p.ntiles = N * p.tiles_per_img;
        set_remap(p);
        const double c = makespan(sh, p, num_cu);
        if (c < best_cost * 0.999) { best_cost = c; best = p; }
    }
    for (int Ra = 1; Ra <= rmax; ++Ra)
        for (int Rb = 1; Rb < Ra; ++Rb) {
            if (H % (Ra + Rb) || tile_lds_bytes(Ra, W) > kInBufBytes) continue;
            Plan p{Ra, Rb, H / (Ra + Rb), 0, 0};
            p.ntiles = 2 * N * p.tiles_per_img;
            set_remap(p);
            const double c = makespan(sh, p, num_cu);
            if (c < best_cost * 0.999) { best_cost = c; best = p; }
        }
    return best;
}

}  // namespace

bool conv3x3s1_supported(const Shape &sh, const void *x, const void *w) {
    const int64_t HW = (int64_t)sh.H * sh.W;
    return sh.ndim == 2 && sh.K == 3 && sh.s == 1 && sh.p == 1 && sh.C % kIcStage == 0 &&
           sh.Co % kOcTile == 0 && sh.W % 8 == 0 && sh.W >= 8 && sh.W <= 64 &&
           (int64_t)sh.C * HW * 2 < (INT64_C(1) << 31) &&            // one image within a buffer range
           (int64_t)kOcTile * HW * 4 < (INT64_C(1) << 31) &&         // one output block within a buffer range
           (int64_t)kOcTile * sh.C * 9 * 2 < (INT64_C(1) << 31) &&
           ((uintptr_t)x % 16) == 0 && ((uintptr_t)w % 16) == 0 && tile_lds_bytes(1, sh.W) <= kInBufBytes;
}

hipError_t launch_conv3x3s1_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w,
                                 const float *bias, float *y, hipStream_t st) {
    static int num_cu = 0;
    if (num_cu == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            num_cu <= 0)
            num_cu = 256;
    }
    // The plan depends only on (N, H, W); remember the last one.
    static int last_n = -1, last_h = -1, last_w = -1;
    static Plan last{};
    if (sh.N != last_n || sh.H != last_h || sh.W != last_w) {
        last = make_plan(sh, slots_for(sh, num_cu));
        last_n = sh.N; last_h = sh.H; last_w = sh.W;
    }
    const Plan pl = last;
    dim3 grid((unsigned)grid_size(pl, slots_for(sh, num_cu)), (unsigned)(sh.Co / kOcTile));
    switch (row_px_for(sh.W)) {
        case 10:
            hipLaunchKernelGGL(conv3x3s1_kernel<10>, grid, dim3(kThreads), 0, st, x, w, bias, y, sh.C,
                               sh.H, sh.W, sh.Co, pl);
            break;
        case 18:
            hipLaunchKernelGGL(conv3x3s1_kernel<18>, grid, dim3(kThreads), 0, st, x, w, bias, y, sh.C,
                               sh.H, sh.W, sh.Co, pl);
            break;
        case 34:
            hipLaunchKernelGGL(conv3x3s1_kernel<34>, grid, dim3(kThreads), 0, st, x, w, bias, y, sh.C,
                               sh.H, sh.W, sh.Co, pl);
            break;
        default:
            hipLaunchKernelGGL(conv3x3s1_kernel<66>, grid, dim3(kThreads), 0, st, x, w, bias, y, sh.C,
                               sh.H, sh.W, sh.Co, pl);
            break;
    }
    return hipGetLastError();
}

}  // namespace convfwd
