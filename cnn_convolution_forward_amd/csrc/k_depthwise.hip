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
// A tile is 32 x TW output positions (TW = 64, or 32 for narrow maps) of one
// input channel c of one image.  Its input patch -- 31*s + d(K-1) + 1 rows by
// (TW-1)*s + d(K-1) + 1 columns, zero outside the input (padding by bounds
// checks) -- is staged in LDS as fp32, consecutive threads on consecutive
// input columns.  Then for each of the M output channels of c a thread owns
// one output column and RB consecutive rows, reads its taps from LDS and the
// K*K weights of the channel (the same for the whole workgroup) through the
// scalar cache, and stores RB fp32 values, consecutive lanes on consecutive
// columns.  The 3x3 stride-1 and stride-2 cases are compiled with constant
// stride and dilation, so the taps shared by neighbouring rows are read once.
//
// Two kernels share that tile body:
//  * multi-tile (the usual one): a workgroup runs several consecutive tiles;
//    the next tile's patch is loaded into registers (16-byte units) while the
//    current tile is computed and stored, into the other of two LDS buffers,
//    with one barrier per tile;
//  * single-tile: one tile per workgroup, the patch loaded in batches; for
//    rows that are not 16-byte aligned (W % 8 != 0 for bf16) or patches too
//    large to prefetch in registers.
#include "conv_internal.h"
#include "mfma_common.h"

namespace convfwd {
namespace {

constexpr int kThreads = 256;
constexpr int kTH = 32;                      // output rows per tile
constexpr int kBatch = 8;                    // element loads in flight per thread (4 for 16-byte units)
constexpr int kMaxPatch = 12 * 1024;         // fp32 patch elements in LDS (48 KB)
constexpr int kMaxPrefetch = 8;              // 16-byte units per thread the multi-tile kernel holds
constexpr int kTilesPerBlock = 8;

template <typename T> __device__ __forceinline__ float ldv(const T *p, int64_t i);
template <> __device__ __forceinline__ float ldv<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldv<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
}

// The patch is staged in units of VEC consecutive input columns: VEC = 1
// (one element) in general, or 16 bytes (8 bf16 / 4 fp32) when W % VEC == 0
// and x is 16-byte aligned, so that a unit is either wholly inside or wholly
// outside [0, W).  Units are read with buffer loads; an offset past the
// resource (kOob) reads 0, so padding needs no branch and a whole batch of
// loads stays in flight together.  raw() loads a unit's bits, put() writes
// them to LDS as fp32.
template <typename T, int VEC> struct Unit;
template <> struct Unit<uint16_t, 1> {
    typedef uint32_t raw_t;
    static __device__ __forceinline__ raw_t raw(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    }
    static __device__ __forceinline__ void put(float *p, raw_t v) { p[0] = __uint_as_float(v << 16); }
};
template <> struct Unit<float, 1> {
    typedef uint32_t raw_t;
    static __device__ __forceinline__ raw_t raw(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    }
    static __device__ __forceinline__ void put(float *p, raw_t v) { p[0] = __uint_as_float(v); }
};
template <> struct Unit<uint16_t, 8> {
    typedef uint4 raw_t;
    static __device__ __forceinline__ raw_t raw(__amdgpu_buffer_rsrc_t r, uint32_t off) { return bload16(r, off, 0); }
    static __device__ __forceinline__ void put(float *p, raw_t q) {
        float4 *d = reinterpret_cast<float4 *>(p);
        d[0] = make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u),
                           __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xffff0000u));
        d[1] = make_float4(__uint_as_float(q.z << 16), __uint_as_float(q.z & 0xffff0000u),
                           __uint_as_float(q.w << 16), __uint_as_float(q.w & 0xffff0000u));
    }
};
template <> struct Unit<float, 4> {
    typedef uint4 raw_t;
    static __device__ __forceinline__ raw_t raw(__amdgpu_buffer_rsrc_t r, uint32_t off) { return bload16(r, off, 0); }
    static __device__ __forceinline__ void put(float *p, raw_t q) {
        *reinterpret_cast<float4 *>(p) =
            make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z), __uint_as_float(q.w));
    }
};

struct DwGeom {
    int TW;              // output tile width (64 or 32); the tile is kTH rows high
    int vec;             // staging unit in elements (1, or 16 bytes' worth)
    int PR, PC;          // patch rows / columns the tile needs
    int shift;           // patch column 0 sits `shift` columns into the first unit
    int CPR, PCP;        // units per patch row; LDS row pitch in elements (CPR * vec)
    int rstep, cstep;    // 256 units = rstep rows + cstep units
    int tiles_w, tiles_h;
};

template <typename T>
__host__ __device__ inline DwGeom dw_geom(const Shape &sh, bool vec_ok) {
    DwGeom g;
    g.TW = sh.Wo > 32 ? 64 : 32;
    g.vec = vec_ok ? 16 / (int)sizeof(T) : 1;
    g.PR = (kTH - 1) * sh.s + (sh.K - 1) * sh.dil + 1;
    g.PC = (g.TW - 1) * sh.s + (sh.K - 1) * sh.dil + 1;
    // every tile starts at input column ow0*s - p with ow0 a multiple of TW,
    // so the first column's offset inside its unit is the same for all tiles
    g.shift = ((-sh.p) % g.vec + g.vec) % g.vec;
    g.CPR = (g.shift + g.PC + g.vec - 1) / g.vec;
    g.PCP = g.CPR * g.vec;
    g.rstep = kThreads / g.CPR;
    g.cstep = kThreads % g.CPR;
    g.tiles_w = (sh.Wo + g.TW - 1) / g.TW;
    g.tiles_h = (sh.Ho + kTH - 1) / kTH;
    return g;
}

// Where tile t (tile column fastest, then tile row, then plane n*C + c) sits.
struct DwTile {
    int64_t plane, n;
    int c, oh0, ow0, ih0, iw0;    // iw0: input column of the first staging unit
};

__device__ __forceinline__ DwTile dw_tile(const Shape &sh, const DwGeom &g, uint32_t t, int S) {
    DwTile d;
    const int tw = (int)(t % (uint32_t)g.tiles_w);
    t /= (uint32_t)g.tiles_w;
    const int th = (int)(t % (uint32_t)g.tiles_h);
    t /= (uint32_t)g.tiles_h;
    d.plane = t;
    d.c = (int)(t % (uint32_t)sh.C);
    d.n = t / (uint32_t)sh.C;
    d.oh0 = th * kTH;
    d.ow0 = tw * g.TW;
    d.ih0 = d.oh0 * S - sh.p;
    d.iw0 = d.ow0 * S - sh.p - g.shift;
    return d;
}

// The tile body: M output channels from the patch in LDS.  Threads outside the
// output skip the work (no early return: callers may have barriers after it).
template <typename T, int KS, int SS, int DS, int RB>
__device__ __forceinline__ void dw_compute(const Shape &sh, const DwGeom &g, const DwTile &d, const float *patch,
                                           const T *__restrict__ w, const float *__restrict__ bias,
                                           float *__restrict__ y) {
    const int K = KS ? KS : sh.K, S = SS ? SS : sh.s, DL = DS ? DS : sh.dil;
    const int M = sh.Co / sh.C;
    const int tid = threadIdx.x;
    const int col = tid % g.TW, strip = tid / g.TW;
    const int ow = d.ow0 + col;
    const int ohs = d.oh0 + strip * RB;
    if (ow >= sh.Wo || ohs >= sh.Ho) return;
    const float *pb = patch + (strip * RB * S) * g.PCP + g.shift + col * S;
    const int64_t oplane = (int64_t)sh.Ho * sh.Wo;

    for (int m = 0; m < M; ++m) {
        const int oc = d.c * M + m;
        const T *wc = w + (int64_t)oc * K * K;
        const float bv = bias ? bias[oc] : 0.f;
        float acc[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) acc[i] = 0.f;
#pragma unroll
        for (int kh = 0; kh < K; ++kh) {
#pragma unroll
            for (int kw = 0; kw < K; ++kw) {
                const float wv = ldv(wc, kh * K + kw);
                const float *pt = pb + (kh * DL) * g.PCP + kw * DL;
#pragma unroll
                for (int i = 0; i < RB; ++i) acc[i] = __builtin_fmaf(pt[i * S * g.PCP], wv, acc[i]);
            }
        }
        // rows past the output go to kOob: the store is dropped, no branch.
        // Optional ReLU, then an fp32 or a bf16 (rounded to nearest even) store.
        const int ob = sh.out_bf16 ? 2 : 4;
        const __amdgpu_buffer_rsrc_t yr =
            make_rsrc((char *)y + (d.n * sh.Co + oc) * oplane * ob, (uint32_t)(oplane * ob));
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const uint32_t o = ohs + i < sh.Ho ? (uint32_t)((ohs + i) * sh.Wo + ow) * (uint32_t)ob : kOob;
            float v = acc[i] + bv;
            if (sh.relu) v = fmaxf(v, 0.f);
            if (sh.out_bf16)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(v), yr, (int)o, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yr, (int)o, 0, 0);
        }
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const void *x, const Shape &sh, int64_t plane,
                                                            int esize) {
    const int64_t hw = (int64_t)sh.H * sh.W;
    return make_rsrc((const char *)x + plane * hw * esize, (uint32_t)(hw * esize));
}

// One tile per workgroup; the patch loaded in batches of NB units.
template <typename T, int KS, int SS, int DS, int RB, int VEC>
__global__ __launch_bounds__(kThreads)
void depthwise_kernel(Shape sh, DwGeom g, const T *__restrict__ x, const T *__restrict__ w,
                      const float *__restrict__ bias, float *__restrict__ y) {
    extern __shared__ __align__(16) float patch[];
    typedef Unit<T, VEC> U;
    const int S = SS ? SS : sh.s;
    const int tid = threadIdx.x;
    const DwTile d = dw_tile(sh, g, blockIdx.x, S);
    const __amdgpu_buffer_rsrc_t xr = plane_rsrc(x, sh, d.plane, sizeof(T));

    // unit tid + 256*i sits at (r, cu), advanced by (rstep, cstep) per step
    constexpr int NB = VEC == 1 ? kBatch : kBatch / 2;
    int r = tid / g.CPR, cu = tid - r * g.CPR;
    for (int base = 0; base < g.PR * g.CPR; base += NB * kThreads) {
        typename U::raw_t v[NB];
        int off[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int ih = d.ih0 + r, iw = d.iw0 + cu * VEC;
            const bool in = r < g.PR && 0 <= ih && ih < sh.H && 0 <= iw && iw < sh.W;
            v[i] = U::raw(xr, in ? (uint32_t)(ih * sh.W + iw) * (uint32_t)sizeof(T) : kOob);
            off[i] = r < g.PR ? r * g.PCP + cu * VEC : -1;
            r += g.rstep;
            cu += g.cstep;
            if (cu >= g.CPR) { cu -= g.CPR; ++r; }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (off[i] >= 0) U::put(patch + off[i], v[i]);
    }
    __syncthreads();
    dw_compute<T, KS, SS, DS, RB>(sh, g, d, patch, w, bias, y);
}

// Tiles [blockIdx.x * nt, +nt) of `tiles`, patch of tile t+1 in flight while
// tile t is computed; two LDS patch buffers.  NU units per thread cover a
// patch (NU * 256 >= PR * CPR).
template <typename T, int KS, int SS, int DS, int RB, int VEC, int NU>
__global__ __launch_bounds__(kThreads)
void depthwise_mt_kernel(Shape sh, DwGeom g, int nt, uint32_t tiles, const T *__restrict__ x,
                         const T *__restrict__ w, const float *__restrict__ bias, float *__restrict__ y) {
    extern __shared__ __align__(16) float patch[];
    typedef Unit<T, VEC> U;
    const int S = SS ? SS : sh.s;
    const int tid = threadIdx.x;
    const int bufsz = g.PR * g.PCP;

    // this thread's units: patch row, first column, LDS offset (-1: none)
    int ur[NU], uc[NU], uo[NU];
    {
        int r = tid / g.CPR, cu = tid - r * g.CPR;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            ur[i] = r;
            uc[i] = cu * VEC;
            uo[i] = r < g.PR ? r * g.PCP + cu * VEC : -1;
            r += g.rstep;
            cu += g.cstep;
            if (cu >= g.CPR) { cu -= g.CPR; ++r; }
        }
    }
    typename U::raw_t v[NU];
    auto fetch = [&](const DwTile &d) {
        const __amdgpu_buffer_rsrc_t xr = plane_rsrc(x, sh, d.plane, sizeof(T));
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int ih = d.ih0 + ur[i], iw = d.iw0 + uc[i];
            const bool in = uo[i] >= 0 && 0 <= ih && ih < sh.H && 0 <= iw && iw < sh.W;
            v[i] = U::raw(xr, in ? (uint32_t)(ih * sh.W + iw) * (uint32_t)sizeof(T) : kOob);
        }
    };

    const uint32_t t0 = blockIdx.x * (uint32_t)nt;
    const uint32_t t1 = t0 + (uint32_t)nt < tiles ? t0 + (uint32_t)nt : tiles;
    DwTile cur = dw_tile(sh, g, t0, S);
    fetch(cur);
    for (uint32_t t = t0; t < t1; ++t) {
        float *buf = patch + ((t - t0) & 1) * bufsz;
#pragma unroll
        for (int i = 0; i < NU; ++i)
            if (uo[i] >= 0) U::put(buf + uo[i], v[i]);
        // the other buffer's last reader (tile t-1) finished before this barrier
        __syncthreads();
        DwTile nxt = cur;
        if (t + 1 < t1) {
            nxt = dw_tile(sh, g, t + 1, S);
            fetch(nxt);
        }
        dw_compute<T, KS, SS, DS, RB>(sh, g, cur, buf, w, bias, y);
        cur = nxt;
    }
}

template <typename T>
bool dw_vec_ok(const Shape &sh, const void *x) {
    return sh.W % (16 / (int)sizeof(T)) == 0 && (uintptr_t)x % 16 == 0;
}

template <typename T, int KS, int SS, int DS, int VEC>
void launch_dw_k(const Shape &sh, const DwGeom &g, const T *x, const T *w, const float *bias, float *y,
                 hipStream_t st) {
    const int64_t tiles = (int64_t)sh.N * sh.C * g.tiles_h * g.tiles_w;
    const size_t lds = (size_t)g.PR * g.PCP * sizeof(float);
    const int units = (g.PR * g.CPR + kThreads - 1) / kThreads;
    // 64 columns: 4 strips of 8 rows; 32 columns: 8 strips of 4 rows
    if constexpr (VEC > 1) {
        if (units <= kMaxPrefetch && 2 * lds <= (size_t)kMaxPatch * 4) {
            const int nt = tiles >= 2048 * kTilesPerBlock ? kTilesPerBlock : (tiles >= 4096 ? 2 : 1);
            const unsigned grid = (unsigned)((tiles + nt - 1) / nt);
#define DW_MT(RB_, NU_)                                                                                        \
    hipLaunchKernelGGL((depthwise_mt_kernel<T, KS, SS, DS, RB_, VEC, NU_>), dim3(grid), dim3(kThreads), 2 * lds, \
                       st, sh, g, nt, (uint32_t)tiles, x, w, bias, y)
            if (g.TW == 64) {
                if (units <= 2) DW_MT(kTH / 4, 2);
                else if (units <= 4) DW_MT(kTH / 4, 4);
                else DW_MT(kTH / 4, 8);
            } else {
                if (units <= 2) DW_MT(kTH / 8, 2);
                else if (units <= 4) DW_MT(kTH / 8, 4);
                else DW_MT(kTH / 8, 8);
            }
#undef DW_MT
            return;
        }
    }
    if (g.TW == 64)
        hipLaunchKernelGGL((depthwise_kernel<T, KS, SS, DS, kTH / 4, VEC>), dim3((unsigned)tiles), dim3(kThreads),
                           lds, st, sh, g, x, w, bias, y);
    else
        hipLaunchKernelGGL((depthwise_kernel<T, KS, SS, DS, kTH / 8, VEC>), dim3((unsigned)tiles), dim3(kThreads),
                           lds, st, sh, g, x, w, bias, y);
}

template <typename T, int VEC>
void launch_dw_v(const Shape &sh, const DwGeom &g, const T *x, const T *w, const float *bias, float *y,
                 hipStream_t st) {
    if (sh.K == 3 && sh.s == 1 && sh.dil == 1)
        launch_dw_k<T, 3, 1, 1, VEC>(sh, g, x, w, bias, y, st);
    else if (sh.K == 3 && sh.s == 2 && sh.dil == 1)
        launch_dw_k<T, 3, 2, 1, VEC>(sh, g, x, w, bias, y, st);
    else if (sh.K == 3)
        launch_dw_k<T, 3, 0, 0, VEC>(sh, g, x, w, bias, y, st);
    else
        launch_dw_k<T, 0, 0, 0, VEC>(sh, g, x, w, bias, y, st);
}

template <typename T>
hipError_t launch_dw(const Shape &sh, const T *x, const T *w, const float *bias, float *y, hipStream_t st) {
    const DwGeom gv = dw_geom<T>(sh, true);
    if (dw_vec_ok<T>(sh, x) && (int64_t)gv.PR * gv.PCP <= kMaxPatch)
        launch_dw_v<T, 16 / sizeof(T)>(sh, gv, x, w, bias, y, st);
    else
        launch_dw_v<T, 1>(sh, dw_geom<T>(sh, false), x, w, bias, y, st);
    return hipGetLastError();
}

}  // namespace

bool depthwise_supported(const Shape &sh) {
    if (sh.ndim != 2 || sh.Cg() != 1 || sh.nhwc) return false;
    // one input or output plane per buffer resource, byte offsets below kOob
    if ((int64_t)sh.H * sh.W * 4 >= (INT64_C(1) << 31) || (int64_t)sh.Ho * sh.Wo * 4 >= (INT64_C(1) << 31))
        return false;
    const DwGeom g = dw_geom<float>(sh, false);          // the element-wise patch, the widest form
    if ((int64_t)g.PR * g.PCP > kMaxPatch) return false;
    const int64_t tiles = (int64_t)sh.N * sh.C * g.tiles_h * g.tiles_w;
    return tiles < (INT64_C(1) << 31);
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
