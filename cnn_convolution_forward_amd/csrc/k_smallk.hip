// k_smallk.hip -- implicit-GEMM convolution for a short reduction
// (C_in * K^dims <= 128: RGB stems, first 3D layers), any K, stride and pad,
// 2D or 3D, bf16 in, fp32 accumulate and out, on the gfx950 matrix cores.
//
// Y = W_row @ X_col ("Why use matrix multiplication for convolution", 2.3)
// with the patch matrix X_col (same page, 2.2) never stored.  A workgroup
// owns TR whole output rows of one (image, output depth): it copies the input
// patch those rows read -- all C_in channels, K_d planes, (TR-1)*s + K rows and
// the columns the taps reach, zero outside the image ("Hand-writing Conv2D",
// 1.2: out-of-range taps read 0) -- into LDS once (for W % 8 == 0: zero fill,
// then in-range input rows copied in 16-byte pieces to a 16-byte aligned
// column origin), together with a table
// koff[k] that gives, for every row k = ((ic*K_d + kd)*K + kh)*K + kw of
// X_col, that tap's offset from a pixel's patch origin.  The X_col column of
// output pixel (r, c) of the tile is then patch[origin(r, c) + koff[k]]: a
// lane gathers its 8 operand values with 8 two-byte LDS reads, and padding
// rows k >= C_in*K^dims point at a zero element.
//
// MFMA: v_mfma_f32_32x32x16_bf16, D[oc][px] = W_row[oc][k] * X_col[k][px]; a
// workgroup covers 64 output channels (two 32-row A operands, staged in LDS
// once) and its waves walk the tile's 32-pixel columns.  Each finished column
// is stored at once -- 32 lanes on 32 consecutive pixels of one channel -- so
// the output, which dominates the traffic (4 * C_out bytes per pixel against
// 2 * C_in * s^dims read), leaves as a continuous stream of full lines.
#include <atomic>

#include "conv_internal.h"
#include "mfma_common.h"

namespace convfwd {
namespace {

constexpr int kOcBlock = 64;            // output channels per workgroup
constexpr int kMaxK = 128;              // C_in * K^dims, padded to 16
constexpr int kPatchElems = 16384;      // LDS patch budget (32 KB)

struct SmallKPlan {
    int TR;          // output rows per tile
    int Rt, Wt;      // patch rows and columns (row pitch)
    int X0;          // patch column of input column 0 (>= pad)
    int vec;         // 1: rows are copied in 16-byte pieces (W % 8 == 0, aligned x, X0 and Wt multiples of 8)
    int E;           // patch elements: C_in*K_d*Rt*Wt input values, then Rt*Wt zeros
    int kg, kpad;    // reduction length and its multiple of 16
    int tiles_h;     // tiles per (image, output depth)
    // reciprocals of the divisors of the prologue's index arithmetic (see
    // div_small): 16-byte pieces per input row, patch rows, K_d, kg
    float inv_cpr, inv_rt, inv_dt, inv_kg;
    float inv_taps, inv_kk, inv_k;      // ... and of K_d*K^2, K^2 and K (the tap table)
};

// Weight rows in LDS: kpad elements plus 8 (16 bytes) of pitch, so that the
// 16-byte operand reads of consecutive rows spread over the banks.
__host__ __device__ constexpr int w_pitch(int kpad) { return kpad + 8; }

// a / b for 0 <= a < 2^20 and 1 <= b < 2^12, with inv_b = 1.0f / b: the
// float quotient is within one of the true one, and one correction step
// makes it exact.  Full-rate instructions only (a 24-bit multiply), where the
// compiler's general 32-bit division takes ~20, several at quarter rate.
__device__ __forceinline__ int div_small(int a, int b, float inv_b) {
    int q = (int)((float)a * inv_b);
    const int r = a - (int)__umul24((unsigned)q, (unsigned)b);
    q += r >= b ? 1 : 0;
    q -= r < 0 ? 1 : 0;
    return q;
}

// KS: reduction steps of 16 (kpad / 16), a template parameter so the weight
// operands take exactly 8 * KS registers.
template <int KS, bool PAIR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KS <= 4 ? 4 : KS <= 6 ? 3 : 2, 8)))
void smallk_kernel(Shape sh, SmallKPlan pl, const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                   const float *__restrict__ bias, float *__restrict__ y) {
    extern __shared__ __align__(16) uint8_t smem[];
    float *bias_s = reinterpret_cast<float *>(smem);                                 // [64]
    uint16_t *koff = reinterpret_cast<uint16_t *>(smem + kOcBlock * 4);              // [kpad]
    uint16_t *ws = reinterpret_cast<uint16_t *>(smem + kOcBlock * 4 + kMaxK * 2);    // [64][w_pitch(kpad)]
    const int WP = w_pitch(pl.kpad);
    uint16_t *patch = ws + kOcBlock * WP;                                             // [E]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // tile -> (n, od, oh0)
    int t = blockIdx.x;
    const int th = t % pl.tiles_h; t /= pl.tiles_h;
    const int od = t % sh.Do;
    const int n = t / sh.Do;
    const int oh0 = th * pl.TR;
    const int rows = min(pl.TR, sh.Ho - oh0);
    const int npx = rows * sh.Wo;
    const int oc0 = blockIdx.y * kOcBlock;

    // ---- stage the patch: line li = (channel, depth, row) holds input row
    // (id, ih) at columns X0 + iw; everything else, and the lines after the
    // C_in*K_d*Rt input lines (the zero region), is zero.  Every global load
    // of the prologue (patch pieces, weights, bias) is issued before the
    // first LDS write, so the workgroup waits for memory once, and the index
    // arithmetic of the 16-byte path, the weights and the tap table avoids
    // general divisions: all workgroups of a launch run this prologue at the
    // same time, before any of them stores an output.
    const int Dt = sh.Kd;
    const int HW = sh.H * sh.W;                                     // < 2^31 (smallk_supported)
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(x + (int64_t)n * sh.C * sh.D * HW, (uint32_t)((int64_t)sh.C * sh.D * HW * 2));
    const int cpr = sh.W / 8;                                       // 16-byte pieces per input row (vec)
    const int pieces = pl.vec ? sh.C * Dt * pl.Rt * cpr : 0;
    const int id0 = od * sh.sd - sh.pd, ih0 = oh0 * sh.s - sh.p;
    constexpr int kPer = 4;                                         // pieces per thread per batch
    uint4 pv[kPer];
    int pdst[kPer];                                                 // LDS element index, or -1
    auto load_pieces = [&](int i0) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = i0 + u * 256 + tid;
            const int li = div_small(i, cpr, pl.inv_cpr), pc = i - li * cpr;
            const int cd = div_small(li, pl.Rt, pl.inv_rt), ry = li - cd * pl.Rt;
            const int c = Dt == 1 ? cd : div_small(cd, Dt, pl.inv_dt), dz = cd - c * Dt;
            const int id = id0 + dz, ih = ih0 + ry;
            const bool ok = i < pieces && id >= 0 && id < sh.D && ih >= 0 && ih < sh.H;
            pdst[u] = ok ? li * pl.Wt + pl.X0 + pc * 8 : -1;
            pv[u] = bload16(xr, ok ? (uint32_t)(((c * sh.D + id) * HW + ih * sh.W + pc * 8) * 2) : kOob, 0);
        }
    };
    auto store_pieces = [&]() {
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            if (pdst[u] >= 0) *reinterpret_cast<uint4 *>(patch + pdst[u]) = pv[u];
    };
    if (pl.vec) load_pieces(0);
    // this workgroup's weight rows are one contiguous run of W_row (oc0 ..
    // oc0 + nch_w - 1, kg each): read flat in 16-byte pieces when the run is
    // 16-byte aligned (as it is for an aligned w), then placed into rows of
    // pitch WP, zero past kg and past C_out, so that an operand is one
    // aligned 16-byte read
    const int nch_w = min(kOcBlock, sh.Co - oc0);
    const int nel = nch_w * pl.kg;
    const uint16_t *wsrc = w + (int64_t)oc0 * pl.kg;
    const bool w16 = ((uintptr_t)wsrc % 16) == 0;
    const int nw16 = w16 ? nel / 8 : 0;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wsrc, (uint32_t)nel * 2);
    constexpr int kWPer = kOcBlock * kMaxK / 8 / 256;               // 16-byte weight pieces per thread (at most)
    uint4 wv[kWPer];
#pragma unroll
    for (int u = 0; u < kWPer; ++u) {
        const int i = u * 256 + tid;
        wv[u] = bload16(wr, i < nw16 ? (uint32_t)i * 16 : kOob, 0);
    }
    const float bias_v = (tid < kOcBlock && bias && oc0 + tid < sh.Co) ? bias[oc0 + tid] : 0.f;

    // zero: the weight rows (padding), and the whole patch when the pieces
    // fill it; then the data goes in
    for (int i = tid; i < kOcBlock * WP / 8; i += 256) reinterpret_cast<uint4 *>(ws)[i] = make_uint4(0, 0, 0, 0);
    if (pl.vec)
        for (int i = tid; i < pl.E / 8; i += 256) reinterpret_cast<uint4 *>(patch)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    if (pl.vec) {
        store_pieces();
        for (int i0 = kPer * 256; i0 < pieces; i0 += kPer * 256) {
            load_pieces(i0);
            store_pieces();
        }
    } else {
        const int lines = (sh.C * Dt + 1) * pl.Rt;
        const uint16_t *xn = x + (int64_t)n * sh.C * sh.D * HW;
        for (int li = wave; li < lines; li += 4) {
            const int ry = li % pl.Rt, cd = li / pl.Rt;
            const int dz = cd % Dt, c = cd / Dt;
            const int id = id0 + dz, ih = ih0 + ry;
            const bool row_ok = c < sh.C && id >= 0 && id < sh.D && ih >= 0 && ih < sh.H;
            const uint16_t *src = xn + ((int64_t)c * sh.D + (row_ok ? id : 0)) * HW + (int64_t)(row_ok ? ih : 0) * sh.W;
            uint16_t *dst = patch + (int64_t)li * pl.Wt;
            for (int cx = lane; cx < pl.Wt; cx += 64) {
                const int iw = cx - pl.X0;
                dst[cx] = (row_ok && iw >= 0 && iw < sh.W) ? src[iw] : (uint16_t)0;
            }
        }
    }
    // weight pieces into their rows: flat element f is (oc, k) = (f / kg, f % kg)
#pragma unroll
    for (int u = 0; u < kWPer; ++u) {
        const int i = u * 256 + tid;
        if (i < nw16) {
            int oc = div_small(8 * i, pl.kg, pl.inv_kg), k = 8 * i - oc * pl.kg;
            const uint32_t v[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ws[oc * WP + k] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                if (++k == pl.kg) { k = 0; ++oc; }
            }
        }
    }
    for (int f = nw16 * 8 + tid; f < nel; f += 256) {
        const int oc = f / pl.kg;
        ws[oc * WP + (f - oc * pl.kg)] = wsrc[f];
    }
    // tap offsets (padding rows k >= kg point at the zero region, which is
    // longer than any pixel origin), bias
    const int KK = sh.K * sh.K, taps = Dt * KK;
    for (int k = tid; k < pl.kpad; k += 256) {
        int off = sh.C * Dt * pl.Rt * pl.Wt;
        if (k < pl.kg) {
            const int ic = div_small(k, taps, pl.inv_taps);
            int r = k - ic * taps;
            const int kd = div_small(r, KK, pl.inv_kk); r -= kd * KK;
            const int kh = div_small(r, sh.K, pl.inv_k), kw = r - kh * sh.K;
            off = ((ic * Dt + kd) * pl.Rt + kh) * pl.Wt + kw;
        }
        koff[k] = (uint16_t)off;
    }
    if (tid < kOcBlock) bias_s[tid] = bias_v;
    __syncthreads();

    const int khalf = 8 * (lane >> 5);
    // A operands: rows ob*32 + lane%32 of the workgroup's block, k = 16s +
    // khalf .. +7 (zero past C_out and past kg)
    uint4 a[2][KS];
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int s = 0; s < KS; ++s)
            a[ob][s] = *reinterpret_cast<const uint4 *>(ws + (ob * 32 + (lane & 31)) * WP + 16 * s + khalf);

    const int64_t plane = sh.out_plane();
    const uint32_t q0 = (uint32_t)(((int64_t)od * sh.Ho + oh0) * sh.Wo);
    // this workgroup's 64 output channels of image n, 32-bit offsets
    const int nch = min(kOcBlock, sh.Co - oc0);
    const int ob_ = sh.out_bf16 ? 2 : 4;                 // output element bytes (bf16 or fp32)
    const __amdgpu_buffer_rsrc_t yr =
        make_rsrc((char *)y + ((int64_t)n * sh.Co + oc0) * plane * ob_, (uint32_t)(nch * plane * ob_));
    const int nfrag = (npx + 31) / 32;
    for (int f = wave; f < nfrag; f += 4) {
        const int p = f * 32 + (lane & 31);
        const int pc = p < npx ? p : npx - 1;
        const int orow = pc / sh.Wo, ocol = pc - orow * sh.Wo;
        const int base = orow * sh.s * pl.Wt + ocol * sh.s - sh.p + pl.X0;
        f32x16_t acc[2];
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ob][r] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 ko = *reinterpret_cast<const uint4 *>(koff + 16 * s + khalf);
            const uint32_t kv[4] = {ko.x, ko.y, ko.z, ko.w};
            uint32_t bw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = patch[base + (kv[e] & 0xffffu)];
                const uint32_t hi = patch[base + (kv[e] >> 16)];
                bw[e] = lo | (hi << 16);
            }
            const uint4 b = make_uint4(bw[0], bw[1], bw[2], bw[3]);
            acc[0] = mfma32x32x16(a[0][s], b, acc[0]);
            acc[1] = mfma32x32x16(a[1][s], b, acc[1]);
        }
        // y = acc + bias: 32 lanes on 32 consecutive pixels of one channel;
        // pixels past the tile and channels past C_out are not stored.  The
        // channel row offset is wave-uniform except for the lane half (4
        // rows), so it splits into soffset + voffset; bias comes from LDS in
        // the loop (volatile: not held in registers across fragments).
        const int hrow = 4 * (lane >> 5);
        if constexpr (PAIR) {
            // bf16, W_out even (which keeps q0, npx and plane even), y 4-byte aligned: lanes 2k, 2k+1 (pixels p, p + 1,
            // consecutive in y and both inside the tile or both past it) swap
            // one value; each stores a pixel pair as one 4-byte word, the even
            // lane channel c, the odd lane channel c + 1
            const uint32_t odd = lane & 1;
            const uint32_t pv2 =
                p < npx ? (q0 + (uint32_t)(p & ~1) + (uint32_t)(hrow + (int)odd) * (uint32_t)plane) * 2u : kOob;
#pragma unroll
            for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    typedef float f32x4v_t __attribute__((ext_vector_type(4)));
                    const f32x4v_t b4 = *reinterpret_cast<const volatile f32x4v_t *>(bias_s + ob * 32 + 8 * g + hrow);
                    const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        const int c = ob * 32 + 8 * g + e;
                        const uint32_t vo = c + hrow + (int)odd < nch ? pv2 : kOob;
                        const int so = (int)((uint32_t)c * (uint32_t)plane * 2u);
                        float va = acc[ob][4 * g + e] + bb[e], vb = acc[ob][4 * g + e + 1] + bb[e + 1];
                        if (sh.relu) {
                            va = fmaxf(va, 0.f);
                            vb = fmaxf(vb, 0.f);
                        }
                        // quad_perm [1, 0, 3, 2]: swap with the neighbouring lane
                        const float got = __int_as_float(
                            __builtin_amdgcn_mov_dpp(__float_as_int(odd ? va : vb), 0xB1, 0xF, 0xF, true));
                        const uint32_t lo = f32_to_bf16_rne(odd ? got : va);
                        const uint32_t hi = f32_to_bf16_rne(odd ? vb : got);
                        __builtin_amdgcn_raw_buffer_store_b32(lo | (hi << 16), yr, (int)vo, so, 0);
                    }
                }
            continue;
        }
        const uint32_t pvo = p < npx ? (q0 + (uint32_t)p + (uint32_t)hrow * (uint32_t)plane) * (uint32_t)ob_ : kOob;
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                typedef float f32x4v_t __attribute__((ext_vector_type(4)));
                const f32x4v_t b4 = *reinterpret_cast<const volatile f32x4v_t *>(bias_s + ob * 32 + 8 * g + hrow);
                const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = ob * 32 + 8 * g + e;             // channel without the lane-half rows
                    const uint32_t vo = c + hrow < nch ? pvo : kOob;
                    const int so = (int)((uint32_t)c * (uint32_t)plane * (uint32_t)ob_);
                    float v = acc[ob][4 * g + e] + bb[e];
                    if (sh.relu) v = fmaxf(v, 0.f);
                    if (sh.out_bf16)
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(v), yr, (int)vo, so, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yr, (int)vo, so, 0);
                }
            }
    }
}

// Patch geometry for TR output rows: row pitch Wt and origin X0 (vec: both
// multiples of 8 and the whole input row fits, so rows copy in 16-byte pieces).
void patch_geom(const Shape &sh, bool vec, int &X0, int &Wt) {
    const int need = (sh.Wo - 1) * sh.s - sh.p + sh.K;          // columns iw < need are read
    if (vec) {
        X0 = (sh.p + 7) / 8 * 8;
        Wt = (X0 + (need > sh.W ? need : sh.W) + 7) / 8 * 8;
    } else {
        X0 = sh.p;
        Wt = X0 + need;
    }
}

int64_t patch_elems(const Shape &sh, int TR, bool vec) {
    int X0, Wt;
    patch_geom(sh, vec, X0, Wt);
    const int64_t Rt = (int64_t)(TR - 1) * sh.s + sh.K;
    return ((int64_t)sh.C * sh.Kd + 1) * Rt * Wt;
}

bool vec_ok(const Shape &sh, const void *x) {
    return sh.W % 8 == 0 && ((uintptr_t)x % 16) == 0 && sh.p <= 8;
}

size_t smem_bytes_for(int kpad, int64_t E) {
    return (size_t)kOcBlock * 4 + kMaxK * 2 + (size_t)kOcBlock * w_pitch(kpad) * 2 + (size_t)E * 2;
}

// Workgroups of smallk_kernel<KS> one CU holds by registers (the occupancy
// query with no LDS; cached per KS), and the device's CUs and LDS per CU.
struct SmallKDevice {
    int cus, lds_per_cu, reg_wgs;
};

SmallKDevice smallk_device(int KS) {
    static std::atomic<int> reg_cache[9];
    SmallKDevice d{256, 160 * 1024, 1};
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) d.cus = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess && v > 0)
            d.lds_per_cu = v;
    }
    int r = reg_cache[KS].load(std::memory_order_relaxed);
    if (r <= 0) {
        int n = 0;
        hipError_t e = hipErrorInvalidValue;
        switch (KS) {
            case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, smallk_kernel<1, false>, 256, 0); break;
            case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, smallk_kernel<2, false>, 256, 0); break;
            case 3: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, smallk_kernel<3, false>, 256, 0); break;
            case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, smallk_kernel<4, false>, 256, 0); break;
            case 5: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, smallk_kernel<5, false>, 256, 0); break;
            case 6: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, smallk_kernel<6, false>, 256, 0); break;
            case 7: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, smallk_kernel<7, false>, 256, 0); break;
            default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, smallk_kernel<8, false>, 256, 0); break;
        }
        r = (e == hipSuccess && n > 0) ? n : 1;
        reg_cache[KS].store(r, std::memory_order_relaxed);
    }
    d.reg_wgs = r;
    return d;
}

// Row tiles: the workgroups of a round run at once, each copying its patch
// (about one output row's worth of time, measured on the stem) and then
// storing its rows, so a launch takes about rounds x (rows per tile + 1)
// row-times.  Among the even splits of a plane whose patch fits the LDS
// budget, take the cheapest (ties: fewer rounds, then more tiles).  A round
// holds CUs x min(register-limited, LDS-limited) workgroups.
SmallKPlan make_smallk_plan(const Shape &sh, bool vec) {
    SmallKPlan pl{};
    pl.kg = (int)sh.kgemm();
    pl.kpad = (pl.kg + 15) / 16 * 16;
    pl.vec = vec ? 1 : 0;
    const SmallKDevice dv = smallk_device(pl.kpad / 16);
    const int64_t planes = (int64_t)sh.N * sh.Do * ((sh.Co + kOcBlock - 1) / kOcBlock);
    int TR = 0;
    int64_t best = -1, best_rounds = 0;
    for (int TRc = sh.Ho; TRc >= 1; --TRc) {
        const int tiles = (sh.Ho + TRc - 1) / TRc;
        if ((sh.Ho + tiles - 1) / tiles != TRc) continue;           // an even split of the plane only
        const int64_t E = patch_elems(sh, TRc, vec);
        if (E > kPatchElems) continue;
        int64_t per_cu = dv.lds_per_cu / (int64_t)smem_bytes_for(pl.kpad, E);
        if (per_cu > dv.reg_wgs) per_cu = dv.reg_wgs;
        if (per_cu < 1) per_cu = 1;
        const int64_t slots = per_cu * dv.cus;
        const int64_t rounds = (planes * tiles + slots - 1) / slots;
        const int64_t cost = rounds * (TRc + 1);
        if (best < 0 || cost < best || (cost == best && rounds <= best_rounds)) {
            best = cost;
            best_rounds = rounds;
            TR = TRc;
        }
    }
    if (TR == 0) TR = 1;                                              // patch_elems(TR = 1) fits (smallk_supported)
    const int tiles = (sh.Ho + TR - 1) / TR;
    pl.TR = TR;
    pl.Rt = (TR - 1) * sh.s + sh.K;
    patch_geom(sh, vec, pl.X0, pl.Wt);
    pl.E = (int)patch_elems(sh, TR, vec);
    pl.tiles_h = tiles;
    pl.inv_cpr = 1.0f / (float)(sh.W / 8 > 0 ? sh.W / 8 : 1);
    pl.inv_rt = 1.0f / (float)pl.Rt;
    pl.inv_dt = 1.0f / (float)sh.Kd;
    pl.inv_kg = 1.0f / (float)pl.kg;
    pl.inv_taps = 1.0f / (float)(sh.Kd * sh.K * sh.K);
    pl.inv_kk = 1.0f / (float)(sh.K * sh.K);
    pl.inv_k = 1.0f / (float)sh.K;
    return pl;
}

size_t smem_bytes(const SmallKPlan &pl) { return smem_bytes_for(pl.kpad, pl.E); }

}  // namespace

bool smallk_supported(const Shape &sh) {
    if (!sh.plain() || sh.nhwc || sh.kgemm() > kMaxK) return false;
    if (patch_elems(sh, 1, false) > kPatchElems) return false;
    if ((int64_t)kOcBlock * sh.out_plane() * 4 >= (INT64_C(1) << 31)) return false;   // one output block per buffer range
    if ((int64_t)sh.C * sh.D * sh.H * sh.W * 2 >= (INT64_C(1) << 31)) return false;   // one input image per buffer range
    return (int64_t)sh.N * sh.Do * sh.Ho < (INT64_C(1) << 31);
}

hipError_t launch_smallk_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias,
                              float *y, hipStream_t st) {
    const bool vec = vec_ok(sh, x) && patch_elems(sh, 1, true) <= kPatchElems;
    const SmallKPlan pl = make_smallk_plan(sh, vec);
    const int64_t tiles = (int64_t)sh.N * sh.Do * pl.tiles_h;
    dim3 grid((unsigned)tiles, (unsigned)((sh.Co + kOcBlock - 1) / kOcBlock));
    // bf16 output stored as pixel pairs (a separate instantiation, so the
    // fp32 kernels carry none of it)
    const bool pair = sh.out_bf16 && sh.Wo % 2 == 0 && ((uintptr_t)y & 3) == 0;
#define SMALLK_LAUNCH(KSV)                                                                                          \
    if (pair)                                                                                                       \
        hipLaunchKernelGGL((smallk_kernel<KSV, true>), grid, dim3(256), smem_bytes(pl), st, sh, pl, x, w, bias, y); \
    else                                                                                                            \
        hipLaunchKernelGGL((smallk_kernel<KSV, false>), grid, dim3(256), smem_bytes(pl), st, sh, pl, x, w, bias, y)
    switch (pl.kpad / 16) {
        case 1: SMALLK_LAUNCH(1); break;
        case 2: SMALLK_LAUNCH(2); break;
        case 3: SMALLK_LAUNCH(3); break;
        case 4: SMALLK_LAUNCH(4); break;
        case 5: SMALLK_LAUNCH(5); break;
        case 6: SMALLK_LAUNCH(6); break;
        case 7: SMALLK_LAUNCH(7); break;
        case 8: SMALLK_LAUNCH(8); break;
        default: return hipErrorInvalidValue;
    }
#undef SMALLK_LAUNCH
    return hipGetLastError();
}

}  // namespace convfwd
