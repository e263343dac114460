/*
 * conv_ref.c -- the oracle: a plain, slow, obviously correct CPU convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the package smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the HIP
 * library: every formula below is written out again from the pages' definitions.
 *
 * Arithmetic: inputs arrive as doubles (bf16 and fp32 values convert to double
 * exactly), every product and sum is formed in IEEE double, summation runs in
 * the plain loop order of the definition, with no blocking or reordering.
 *
 * Citations name the page and its section:
 *   [Hand-writing Conv2D, 1.1]  the index map y[n][oc][oh][ow] = bias[oc] +
 *        sum over (ic, kh, kw) of x[n][ic][oh*s+kh-p][ow*s+kw-p] * w[oc][ic][kh][kw]
 *        and the output size floor((H + 2p - K)/s) + 1.
 *   [Hand-writing Conv2D, 1.2]  padding by bounds checks: a tap whose input
 *        coordinate falls outside [0, H) x [0, W) contributes nothing.
 *   [Why use matrix multiplication for convolution, 2.2]  the X_col layout:
 *        row = (ic, kh, kw) flattened, column = output position, width fastest.
 *   [Why use matrix multiplication for convolution, 3.1]  column index
 *        n*(H_out*W_out) + oh*W_out + ow.
 *   [PyTorch tensor products and conv2d/conv3d dimension semantics, 5.1, 5.2]
 *        NCDHW input, (C_out, C_in, kD, kH, kW) weights, the same size formula
 *        applied independently to D, H and W.
 *
 * Besides y, each convolution returns S = sum over the same taps of |x * w|
 * (bias excluded), the scale against which a low-precision result is judged.
 *
 * Parity pins live in tests/test_oracle_pins.py (plain convolution),
 * tests/test_oracle_pins_general.py (dilation and groups),
 * tests/test_oracle_pins_backward.py (gradients) and
 * tests/test_oracle_pins_epilogue.py (ReLU, bf16 output, channels-last) and
 * tests/test_oracle_pins_winograd.py (Winograd F(2x2,3x3)); every function here
 * is pinned.
 */
#include <stdint.h>
#include <stdlib.h>
#include <stddef.h>
#include <string.h>
#include <math.h>
#include <time.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Output length along one spatial dimension: floor((in + 2p - k)/s) + 1
 * [Hand-writing Conv2D, 1.1].  Returns -1 when the window does not fit even
 * once (in + 2p < k) or a parameter is out of range; C integer division
 * truncates toward zero, so the negative numerator is rejected explicitly
 * rather than silently yielding 1 [Conv2d from the official docs, 3.2]. */
int64_t oracle_out_dim(int64_t in, int64_t k, int64_t s, int64_t p)
{
    if (in < 1 || k < 1 || s < 1 || p < 0) return -1;
    int64_t num = in + 2 * p - k;
    if (num < 0) return -1;
    return num / s + 1;          /* num >= 0 here, so '/' is floor */
}

/* bf16 bit pattern -> double, exactly: a bf16 is the top 16 bits of a binary32. */
void oracle_bf16_to_f64(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t bits = ((uint32_t)src[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        dst[i] = (double)f;
    }
}

/* binary32 -> double, exactly. */
void oracle_f32_to_f64(const float *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = (double)src[i];
}

/* One output element of a 3D convolution (2D is the case D = 1, kd range {0}).
 * x: (N, C, D, H, W), w: (Co, C, Kd, K, K); kd_size = 1 and pd = 0 for 2D.
 * Loop order is the definition's: ic, then kd, kh, kw. */
static void one_output(const double *x, const double *w, int64_t n, int64_t oc,
                       int64_t od, int64_t oh, int64_t ow,
                       int64_t C, int64_t D, int64_t H, int64_t W,
                       int64_t Kd, int64_t K, int64_t s, int64_t sd,
                       int64_t p, int64_t pd, double *acc_out, double *S_out)
{
    double acc = 0.0, S = 0.0;
    for (int64_t ic = 0; ic < C; ++ic) {
        for (int64_t kd = 0; kd < Kd; ++kd) {
            int64_t id = od * sd + kd - pd;
            if (!(0 <= id && id < D)) continue;          /* [Hand-writing Conv2D, 1.2] */
            for (int64_t kh = 0; kh < K; ++kh) {
                int64_t ih = oh * s + kh - p;
                if (!(0 <= ih && ih < H)) continue;
                for (int64_t kw = 0; kw < K; ++kw) {
                    int64_t iw = ow * s + kw - p;
                    if (!(0 <= iw && iw < W)) continue;
                    double xv = x[(((n * C + ic) * D + id) * H + ih) * W + iw];
                    double wv = w[(((oc * C + ic) * Kd + kd) * K + kh) * K + kw];
                    double t = xv * wv;
                    acc += t;
                    S += fabs(t);
                }
            }
        }
    }
    *acc_out = acc;
    *S_out = S;
}

/* Full 2D convolution, NCHW x OIHW -> NCHW [Hand-writing Conv2D, 1.1 and 2.1].
 * bias may be NULL (no bias).  S may be NULL.  Returns 0, or -1 on bad shape. */
int oracle_conv2d(const double *x, const double *w, const double *bias,
                  double *y, double *S,
                  int64_t N, int64_t C, int64_t H, int64_t W,
                  int64_t Co, int64_t K, int64_t s, int64_t p)
{
    int64_t Ho = oracle_out_dim(H, K, s, p), Wo = oracle_out_dim(W, K, s, p);
    if (Ho < 0 || Wo < 0 || N < 1 || C < 1 || Co < 1) return -1;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t oc = 0; oc < Co; ++oc)
            for (int64_t oh = 0; oh < Ho; ++oh)
                for (int64_t ow = 0; ow < Wo; ++ow) {
                    double acc, sa;
                    one_output(x, w, n, oc, 0, oh, ow, C, 1, H, W, 1, K, s, 1, p, 0, &acc, &sa);
                    int64_t o = ((n * Co + oc) * Ho + oh) * Wo + ow;
                    y[o] = acc + (bias ? bias[oc] : 0.0);
                    if (S) S[o] = sa;
                }
    return 0;
}

/* Full 3D convolution, NCDHW x (Co, C, K, K, K) -> NCDHW, one K, s, p for all
 * three dimensions [PyTorch tensor products and conv2d/conv3d dimension
 * semantics, 5.1 and 5.2]. */
int oracle_conv3d(const double *x, const double *w, const double *bias,
                  double *y, double *S,
                  int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                  int64_t Co, int64_t K, int64_t s, int64_t p)
{
    int64_t Do = oracle_out_dim(D, K, s, p);
    int64_t Ho = oracle_out_dim(H, K, s, p), Wo = oracle_out_dim(W, K, s, p);
    if (Do < 0 || Ho < 0 || Wo < 0 || N < 1 || C < 1 || Co < 1) return -1;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t oc = 0; oc < Co; ++oc)
            for (int64_t od = 0; od < Do; ++od)
                for (int64_t oh = 0; oh < Ho; ++oh)
                    for (int64_t ow = 0; ow < Wo; ++ow) {
                        double acc, sa;
                        one_output(x, w, n, oc, od, oh, ow, C, D, H, W, K, K, s, s, p, p, &acc, &sa);
                        int64_t o = (((n * Co + oc) * Do + od) * Ho + oh) * Wo + ow;
                        y[o] = acc + (bias ? bias[oc] : 0.0);
                        if (S) S[o] = sa;
                    }
    return 0;
}

/* Selected outputs only, for checks at sizes where the full tensor is too slow.
 * idx holds flat NC(D)HW output indices; ndim is 2 or 3 (D ignored for 2). */
int oracle_conv_points(int ndim, const double *x, const double *w, const double *bias,
                       const int64_t *idx, int64_t npts, double *y, double *S,
                       int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                       int64_t Co, int64_t K, int64_t s, int64_t p)
{
    int64_t Dd = (ndim == 3) ? D : 1, Kd = (ndim == 3) ? K : 1;
    int64_t sd = (ndim == 3) ? s : 1, pd = (ndim == 3) ? p : 0;
    int64_t Do = (ndim == 3) ? oracle_out_dim(D, K, s, p) : 1;
    int64_t Ho = oracle_out_dim(H, K, s, p), Wo = oracle_out_dim(W, K, s, p);
    if ((ndim != 2 && ndim != 3) || Do < 0 || Ho < 0 || Wo < 0) return -1;
    int64_t total = N * Co * Do * Ho * Wo;
    for (int64_t i = 0; i < npts; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -1;
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t o = idx[i];
        int64_t ow = o % Wo; o /= Wo;
        int64_t oh = o % Ho; o /= Ho;
        int64_t od = o % Do; o /= Do;
        int64_t oc = o % Co; o /= Co;
        int64_t n = o;
        double acc, sa;
        one_output(x, w, n, oc, od, oh, ow, C, Dd, H, W, Kd, K, s, sd, p, pd, &acc, &sa);
        y[i] = acc + (bias ? bias[oc] : 0.0);
        if (S) S[i] = sa;
    }
    return 0;
}

/* Explicit im2col, 2D [Why use matrix multiplication for convolution, 2.2 and
 * 3.1]: col has shape (C*K*K, N*Ho*Wo), row r = (ic*K + kh)*K + kw, column
 * j = n*Ho*Wo + oh*Wo + ow; an out-of-range tap is 0 (zero padding). */
int oracle_im2col2d(const double *x, double *col,
                    int64_t N, int64_t C, int64_t H, int64_t W,
                    int64_t K, int64_t s, int64_t p)
{
    int64_t Ho = oracle_out_dim(H, K, s, p), Wo = oracle_out_dim(W, K, s, p);
    if (Ho < 0 || Wo < 0) return -1;
    int64_t cols = N * Ho * Wo;
    for (int64_t ic = 0; ic < C; ++ic)
        for (int64_t kh = 0; kh < K; ++kh)
            for (int64_t kw = 0; kw < K; ++kw) {
                int64_t r = (ic * K + kh) * K + kw;
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t oh = 0; oh < Ho; ++oh)
                        for (int64_t ow = 0; ow < Wo; ++ow) {
                            int64_t ih = oh * s + kh - p, iw = ow * s + kw - p;
                            double v = 0.0;
                            if (0 <= ih && ih < H && 0 <= iw && iw < W)
                                v = x[((n * C + ic) * H + ih) * W + iw];
                            col[r * cols + (n * Ho + oh) * Wo + ow] = v;
                        }
            }
    return 0;
}

/* Explicit im2col, 3D: row r = ((ic*K + kd)*K + kh)*K + kw, column
 * j = ((n*Do + od)*Ho + oh)*Wo + ow. */
int oracle_im2col3d(const double *x, double *col,
                    int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                    int64_t K, int64_t s, int64_t p)
{
    int64_t Do = oracle_out_dim(D, K, s, p);
    int64_t Ho = oracle_out_dim(H, K, s, p), Wo = oracle_out_dim(W, K, s, p);
    if (Do < 0 || Ho < 0 || Wo < 0) return -1;
    int64_t cols = N * Do * Ho * Wo;
    for (int64_t ic = 0; ic < C; ++ic)
      for (int64_t kd = 0; kd < K; ++kd)
        for (int64_t kh = 0; kh < K; ++kh)
          for (int64_t kw = 0; kw < K; ++kw) {
            int64_t r = ((ic * K + kd) * K + kh) * K + kw;
            for (int64_t n = 0; n < N; ++n)
              for (int64_t od = 0; od < Do; ++od)
                for (int64_t oh = 0; oh < Ho; ++oh)
                  for (int64_t ow = 0; ow < Wo; ++ow) {
                    int64_t id = od * s + kd - p, ih = oh * s + kh - p, iw = ow * s + kw - p;
                    double v = 0.0;
                    if (0 <= id && id < D && 0 <= ih && ih < H && 0 <= iw && iw < W)
                        v = x[(((n * C + ic) * D + id) * H + ih) * W + iw];
                    col[r * cols + ((n * Do + od) * Ho + oh) * Wo + ow] = v;
                  }
          }
    return 0;
}

/* Plain matrix product C (M x Nn) = A (M x Kk) @ B (Kk x Nn), row-major, fp64,
 * the GEMM step Y = W_row @ X_col [Why use matrix multiplication for
 * convolution, 2.3]. */
void oracle_matmul(const double *A, const double *B, double *Cm,
                   int64_t M, int64_t Kk, int64_t Nn)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < Nn; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < Kk; ++k) acc += A[i * Kk + k] * B[k * Nn + j];
            Cm[i * Nn + j] = acc;
        }
}

/* ---- dilation and groups ----------------------------------------------------
 *
 *   [PyTorch tensor products and conv2d/conv3d dimension semantics, 4.2]
 *        with dilation d the taps of one window sit d apart, so a window spans
 *        d(K-1)+1 input positions and out = floor((in + 2p - d(K-1) - 1)/s) + 1
 *        (also [Conv2d from the official docs, 3.2 and 3.3]).
 *   [PyTorch tensor products and conv2d/conv3d dimension semantics, 4.3]
 *        groups g: C_in and C_out are each cut into g equal consecutive blocks;
 *        output block i reads input block i only; the weight's second extent is
 *        C_in/g; g = C_in is the depthwise case ([Conv2d from the official
 *        docs, 3.4] gives the same rule).
 *   The depth dimension of a 3D problem takes the same K, s, p and d
 *   ([PyTorch tensor products and conv2d/conv3d dimension semantics, 5.2]).
 */

/* Output length with dilation d; -1 when a parameter is out of range or the
 * dilated window never fits. */
int64_t oracle_out_dim_dilated(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d)
{
    if (in < 1 || k < 1 || s < 1 || p < 0 || d < 1) return -1;
    int64_t span = d * (k - 1) + 1;
    int64_t room = in + 2 * p - span;
    if (room < 0) return -1;
    return room / s + 1;
}

/* Geometry of one general problem; 2D is carried with Dd = 1 and a depth
 * kernel of one tap. */
typedef struct {
    int64_t N, C, Dd, H, W, Co, G;
    int64_t Kz, K;          /* depth taps (1 in 2D), in-plane taps */
    int64_t s, p, d;        /* in-plane stride, pad, dilation      */
    int64_t sz, pz, dz;     /* depth stride, pad, dilation         */
    int64_t Do, Ho, Wo;
} gen_geom;

static int gen_geom_make(gen_geom *g, int ndim, int64_t N, int64_t C, int64_t D, int64_t H,
                         int64_t W, int64_t Co, int64_t K, int64_t s, int64_t p, int64_t d,
                         int64_t G)
{
    if (ndim != 2 && ndim != 3) return -1;
    if (N < 1 || C < 1 || Co < 1 || G < 1 || C % G != 0 || Co % G != 0) return -1;
    g->N = N; g->C = C; g->H = H; g->W = W; g->Co = Co; g->G = G;
    g->K = K; g->s = s; g->p = p; g->d = d;
    if (ndim == 3) {
        g->Dd = D; g->Kz = K; g->sz = s; g->pz = p; g->dz = d;
        g->Do = oracle_out_dim_dilated(D, K, s, p, d);
    } else {
        g->Dd = 1; g->Kz = 1; g->sz = 1; g->pz = 0; g->dz = 1;
        g->Do = 1;
    }
    g->Ho = oracle_out_dim_dilated(H, K, s, p, d);
    g->Wo = oracle_out_dim_dilated(W, K, s, p, d);
    if (g->Do < 0 || g->Ho < 0 || g->Wo < 0) return -1;
    return 0;
}

/* One output element: output channel oc belongs to group oc / (Co/G) and sums
 * over the C/G input channels of that group, the weight holding C/G input
 * channels per filter.  Tap (kz, kh, kw) reads input (od*sz + kz*dz - pz,
 * oh*s + kh*d - p, ow*s + kw*d - p); outside the input it adds nothing. */
static void gen_one(const gen_geom *g, const double *x, const double *w, int64_t n, int64_t oc,
                    int64_t od, int64_t oh, int64_t ow, double *acc_out, double *S_out)
{
    const int64_t Cg = g->C / g->G, Cog = g->Co / g->G;
    const int64_t grp = oc / Cog;
    double acc = 0.0, S = 0.0;
    for (int64_t j = 0; j < Cg; ++j) {
        const int64_t ic = grp * Cg + j;
        for (int64_t kz = 0; kz < g->Kz; ++kz) {
            const int64_t iz = od * g->sz + kz * g->dz - g->pz;
            if (iz < 0 || iz >= g->Dd) continue;
            for (int64_t kh = 0; kh < g->K; ++kh) {
                const int64_t iy = oh * g->s + kh * g->d - g->p;
                if (iy < 0 || iy >= g->H) continue;
                for (int64_t kw = 0; kw < g->K; ++kw) {
                    const int64_t ix = ow * g->s + kw * g->d - g->p;
                    if (ix < 0 || ix >= g->W) continue;
                    const double xv = x[(((n * g->C + ic) * g->Dd + iz) * g->H + iy) * g->W + ix];
                    const double wv = w[(((oc * Cg + j) * g->Kz + kz) * g->K + kh) * g->K + kw];
                    const double prod = xv * wv;
                    acc += prod;
                    S += fabs(prod);
                }
            }
        }
    }
    *acc_out = acc;
    *S_out = S;
}

/* Full 2D or 3D convolution with dilation d and groups G.  x: (N, C, [D,] H, W),
 * w: (Co, C/G, K, K[, K]), y and S: (N, Co, [Do,] Ho, Wo).  bias and S may be
 * NULL.  Returns 0, or -1 on a bad shape. */
int oracle_conv_general(int ndim, const double *x, const double *w, const double *bias,
                        double *y, double *S,
                        int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                        int64_t Co, int64_t K, int64_t s, int64_t p, int64_t d, int64_t G)
{
    gen_geom g;
    if (gen_geom_make(&g, ndim, N, C, D, H, W, Co, K, s, p, d, G) != 0) return -1;
    const int64_t plane = g.Do * g.Ho * g.Wo;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t oc = 0; oc < Co; ++oc)
            for (int64_t q = 0; q < plane; ++q) {
                const int64_t ow = q % g.Wo, oh = (q / g.Wo) % g.Ho, od = q / (g.Wo * g.Ho);
                double acc, sa;
                gen_one(&g, x, w, n, oc, od, oh, ow, &acc, &sa);
                const int64_t o = (n * Co + oc) * plane + q;
                y[o] = acc + (bias ? bias[oc] : 0.0);
                if (S) S[o] = sa;
            }
    return 0;
}

/* The same at the flat output indices idx[0..npts) only. */
int oracle_conv_general_points(int ndim, const double *x, const double *w, const double *bias,
                               const int64_t *idx, int64_t npts, double *y, double *S,
                               int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                               int64_t Co, int64_t K, int64_t s, int64_t p, int64_t d, int64_t G)
{
    gen_geom g;
    if (gen_geom_make(&g, ndim, N, C, D, H, W, Co, K, s, p, d, G) != 0) return -1;
    const int64_t plane = g.Do * g.Ho * g.Wo, total = N * Co * plane;
    for (int64_t i = 0; i < npts; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -1;
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t q = idx[i] % plane, oc = (idx[i] / plane) % Co, n = idx[i] / (plane * Co);
        const int64_t ow = q % g.Wo, oh = (q / g.Wo) % g.Ho, od = q / (g.Wo * g.Ho);
        double acc, sa;
        gen_one(&g, x, w, n, oc, od, oh, ow, &acc, &sa);
        y[i] = acc + (bias ? bias[oc] : 0.0);
        if (S) S[i] = sa;
    }
    return 0;
}

/* Explicit im2col with dilation, 2D or 3D [Why use matrix multiplication for
 * convolution, 2.2 and 3.1, with the dilated tap offsets above].  col has
 * C*K^ndim rows, row ((ic*Kz + kz)*K + kh)*K + kw, and N*Do*Ho*Wo columns in
 * output order; an out-of-range tap is 0.  Groups do not change X_col: group i
 * multiplies its own block of C/G * K^ndim consecutive rows. */
int oracle_im2col_dilated(int ndim, const double *x, double *col,
                          int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                          int64_t K, int64_t s, int64_t p, int64_t d)
{
    gen_geom g;
    if (gen_geom_make(&g, ndim, N, C, D, H, W, 1, K, s, p, d, 1) != 0) return -1;
    const int64_t plane = g.Do * g.Ho * g.Wo, cols = N * plane;
    for (int64_t ic = 0; ic < C; ++ic)
      for (int64_t kz = 0; kz < g.Kz; ++kz)
        for (int64_t kh = 0; kh < K; ++kh)
          for (int64_t kw = 0; kw < K; ++kw) {
            const int64_t r = ((ic * g.Kz + kz) * K + kh) * K + kw;
            for (int64_t n = 0; n < N; ++n)
              for (int64_t q = 0; q < plane; ++q) {
                const int64_t ow = q % g.Wo, oh = (q / g.Wo) % g.Ho, od = q / (g.Wo * g.Ho);
                const int64_t iz = od * g.sz + kz * g.dz - g.pz;
                const int64_t iy = oh * s + kh * d - p, ix = ow * s + kw * d - p;
                double v = 0.0;
                if (0 <= iz && iz < g.Dd && 0 <= iy && iy < H && 0 <= ix && ix < W)
                    v = x[(((n * C + ic) * g.Dd + iz) * H + iy) * W + ix];
                col[r * cols + n * plane + q] = v;
              }
          }
    return 0;
}

/* ---- backward: db, dW, dx -------------------------------------------------
 *
 *   [Hand-writing Conv2D, 5.1]  with upstream gradient dout (the shape of y):
 *        db[oc] = sum over n, oh, ow of dout[n][oc][oh][ow];
 *        dW[oc][ic][kh][kw] = sum over n, oh, ow of dout[n][oc][oh][ow] times
 *            the input the tap read, x[n][ic][oh*s + kh - p][ow*s + kw - p]
 *            (taps outside the input add nothing);
 *        dx scatters each dout[n][oc][oh][ow] * w[oc][ic][kh][kw] back onto
 *            the input position that tap read, accumulating (several windows
 *            cover one input).
 *   [Hand-writing Conv2D, 5.2]  the same loop computes dW and dx, since they
 *        visit the same input coordinates; written here over the general
 *        geometry (dilation d, groups G, 3D) of the forward functions above.
 *   [Why use matrix multiplication for convolution, 3.3]  the same results as
 *        dW_row = dout_col @ X_col^T and dx = col2im(W_row^T @ dout_col); see
 *        oracle_col2im_dilated below.
 * Besides the gradients, S_dx, S_dw and S_db hold the sums of the magnitudes
 * of the same products (|w * dout|, |dout * x|, |dout|): the scale against
 * which a low-precision result is judged.  Any of the outputs may be NULL.
 */
int oracle_conv_backward(int ndim, const double *x, const double *w, const double *dout,
                         double *dx, double *dw, double *db,
                         double *S_dx, double *S_dw, double *S_db,
                         int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                         int64_t Co, int64_t K, int64_t s, int64_t p, int64_t d, int64_t G)
{
    gen_geom g;
    if (gen_geom_make(&g, ndim, N, C, D, H, W, Co, K, s, p, d, G) != 0) return -1;
    const int64_t Cg = C / G, Cog = Co / G;
    const int64_t nx = N * C * g.Dd * H * W, nw = Co * Cg * g.Kz * K * K;
    for (int64_t i = 0; i < nx; ++i) { if (dx) dx[i] = 0.0; if (S_dx) S_dx[i] = 0.0; }
    for (int64_t i = 0; i < nw; ++i) { if (dw) dw[i] = 0.0; if (S_dw) S_dw[i] = 0.0; }
    for (int64_t oc = 0; oc < Co; ++oc) { if (db) db[oc] = 0.0; if (S_db) S_db[oc] = 0.0; }
    /* Sequential on purpose: dx and dW are accumulated from many outputs. */
    for (int64_t n = 0; n < N; ++n)
      for (int64_t oc = 0; oc < Co; ++oc) {
        const int64_t grp = oc / Cog;
        for (int64_t od = 0; od < g.Do; ++od)
          for (int64_t oh = 0; oh < g.Ho; ++oh)
            for (int64_t ow = 0; ow < g.Wo; ++ow) {
              const double gout = dout[(((n * Co + oc) * g.Do + od) * g.Ho + oh) * g.Wo + ow];
              if (db) db[oc] += gout;
              if (S_db) S_db[oc] += fabs(gout);
              for (int64_t j = 0; j < Cg; ++j) {
                const int64_t ic = grp * Cg + j;
                for (int64_t kz = 0; kz < g.Kz; ++kz) {
                  const int64_t iz = od * g.sz + kz * g.dz - g.pz;
                  if (iz < 0 || iz >= g.Dd) continue;
                  for (int64_t kh = 0; kh < K; ++kh) {
                    const int64_t iy = oh * s + kh * d - p;
                    if (iy < 0 || iy >= H) continue;
                    for (int64_t kw = 0; kw < K; ++kw) {
                      const int64_t ix = ow * s + kw * d - p;
                      if (ix < 0 || ix >= W) continue;
                      const int64_t xi = (((n * C + ic) * g.Dd + iz) * H + iy) * W + ix;
                      const int64_t wi = (((oc * Cg + j) * g.Kz + kz) * K + kh) * K + kw;
                      if (dw) dw[wi] += gout * x[xi];
                      if (S_dw) S_dw[wi] += fabs(gout * x[xi]);
                      if (dx) dx[xi] += w[wi] * gout;
                      if (S_dx) S_dx[xi] += fabs(w[wi] * gout);
                    }
                  }
                }
              }
            }
      }
    return 0;
}

/* The gradients at chosen points, in gather form, for checks at sizes where
 * the scatter loop above is too slow.  Same definitions [Hand-writing Conv2D,
 * 5.1], each element summed on its own:
 *   dw at flat index idx of (Co, C/G, Kz, K, K): sum over n and every output
 *     position o of dout[n][oc][o] * x[n][ic][o*s + k*d - p] (in range);
 *   dx at flat index idx of (N, C, Dd, H, W): sum over the group's output
 *     channels and the taps k for which (i + p - k*d) is a multiple of s and
 *     o = (i + p - k*d)/s is an output position, of w[oc][j][k] * dout[n][oc][o].
 * S_* as in oracle_conv_backward.  Returns -1 on a bad shape or index. */
int oracle_conv_backward_points(int ndim, const double *x, const double *w, const double *dout,
                                const int64_t *dw_idx, int64_t n_dw, double *dw, double *S_dw,
                                const int64_t *dx_idx, int64_t n_dx, double *dx, double *S_dx,
                                int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                                int64_t Co, int64_t K, int64_t s, int64_t p, int64_t d, int64_t G)
{
    gen_geom g;
    if (gen_geom_make(&g, ndim, N, C, D, H, W, Co, K, s, p, d, G) != 0) return -1;
    const int64_t Cg = C / G, Cog = Co / G;
    const int64_t nw = Co * Cg * g.Kz * K * K, nx = N * C * g.Dd * H * W;
    for (int64_t i = 0; i < n_dw; ++i) if (dw_idx[i] < 0 || dw_idx[i] >= nw) return -1;
    for (int64_t i = 0; i < n_dx; ++i) if (dx_idx[i] < 0 || dx_idx[i] >= nx) return -1;
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_dw; ++i) {
        int64_t r = dw_idx[i];
        const int64_t kw = r % K; r /= K;
        const int64_t kh = r % K; r /= K;
        const int64_t kz = r % g.Kz; r /= g.Kz;
        const int64_t j = r % Cg;
        const int64_t oc = r / Cg;
        const int64_t ic = (oc / Cog) * Cg + j;
        double acc = 0.0, S = 0.0;
        for (int64_t n = 0; n < N; ++n)
          for (int64_t od = 0; od < g.Do; ++od) {
            const int64_t iz = od * g.sz + kz * g.dz - g.pz;
            if (iz < 0 || iz >= g.Dd) continue;
            for (int64_t oh = 0; oh < g.Ho; ++oh) {
              const int64_t iy = oh * s + kh * d - p;
              if (iy < 0 || iy >= H) continue;
              for (int64_t ow = 0; ow < g.Wo; ++ow) {
                const int64_t ix = ow * s + kw * d - p;
                if (ix < 0 || ix >= W) continue;
                const double term = dout[(((n * Co + oc) * g.Do + od) * g.Ho + oh) * g.Wo + ow] *
                                 x[(((n * C + ic) * g.Dd + iz) * H + iy) * W + ix];
                acc += term;
                S += fabs(term);
              }
            }
          }
        dw[i] = acc;
        if (S_dw) S_dw[i] = S;
    }
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n_dx; ++i) {
        int64_t r = dx_idx[i];
        const int64_t ix = r % W; r /= W;
        const int64_t iy = r % H; r /= H;
        const int64_t iz = r % g.Dd; r /= g.Dd;
        const int64_t ic = r % C;
        const int64_t n = r / C;
        const int64_t grp = ic / Cg, j = ic % Cg;
        double acc = 0.0, S = 0.0;
        for (int64_t ocl = 0; ocl < Cog; ++ocl) {
          const int64_t oc = grp * Cog + ocl;
          for (int64_t kz = 0; kz < g.Kz; ++kz) {
            const int64_t tz = iz + g.pz - kz * g.dz;
            if (tz < 0 || tz % g.sz != 0 || tz / g.sz >= g.Do) continue;
            for (int64_t kh = 0; kh < K; ++kh) {
              const int64_t ty = iy + p - kh * d;
              if (ty < 0 || ty % s != 0 || ty / s >= g.Ho) continue;
              for (int64_t kw = 0; kw < K; ++kw) {
                const int64_t tx = ix + p - kw * d;
                if (tx < 0 || tx % s != 0 || tx / s >= g.Wo) continue;
                const double term = w[(((oc * Cg + j) * g.Kz + kz) * K + kh) * K + kw] *
                                 dout[(((n * Co + oc) * g.Do + tz / g.sz) * g.Ho + ty / s) * g.Wo + tx / s];
                acc += term;
                S += fabs(term);
              }
            }
          }
        }
        dx[i] = acc;
        if (S_dx) S_dx[i] = S;
    }
    return 0;
}

/* col2im, the adjoint of oracle_im2col_dilated [Why use matrix multiplication
 * for convolution, 3.3]: every entry of col (C*K^ndim rows, N*Do*Ho*Wo
 * columns, the im2col layout) is added onto the input position its tap read;
 * entries whose tap fell in the padding are dropped (the page pads, adds,
 * then crops the padding away, which is the same).  dx has x's shape. */
int oracle_col2im_dilated(int ndim, const double *col, double *dx,
                          int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                          int64_t K, int64_t s, int64_t p, int64_t d)
{
    gen_geom g;
    if (gen_geom_make(&g, ndim, N, C, D, H, W, 1, K, s, p, d, 1) != 0) return -1;
    const int64_t plane = g.Do * g.Ho * g.Wo, cols = N * plane;
    for (int64_t i = 0; i < N * C * g.Dd * H * W; ++i) dx[i] = 0.0;
    for (int64_t ic = 0; ic < C; ++ic)
      for (int64_t kz = 0; kz < g.Kz; ++kz)
        for (int64_t kh = 0; kh < K; ++kh)
          for (int64_t kw = 0; kw < K; ++kw) {
            const int64_t r = ((ic * g.Kz + kz) * K + kh) * K + kw;
            for (int64_t n = 0; n < N; ++n)
              for (int64_t q = 0; q < plane; ++q) {
                const int64_t ow = q % g.Wo, oh = (q / g.Wo) % g.Ho, od = q / (g.Wo * g.Ho);
                const int64_t iz = od * g.sz + kz * g.dz - g.pz;
                const int64_t iy = oh * s + kh * d - p, ix = ow * s + kw * d - p;
                if (0 <= iz && iz < g.Dd && 0 <= iy && iy < H && 0 <= ix && ix < W)
                    dx[(((n * C + ic) * g.Dd + iz) * H + iy) * W + ix] += col[r * cols + n * plane + q];
              }
          }
    return 0;
}

/* ---- output epilogue and channels-last layout -----------------------------
 *
 * Rectification: out = max(y, 0) (the ReLU that follows the convolution in
 * [PyTorch tensor products and conv2d/conv3d dimension semantics, 6.2]).
 * bf16 output: y rounded to the nearest value with an 8-bit significand, ties
 * to the even significand (IEEE 754 round-to-nearest-even applied to bfloat16,
 * the top 16 bits of a binary32).  Values are finite here; zero stays zero.
 */
double oracle_round_bf16(double v)
{
    if (v == 0.0 || !isfinite(v)) return v;
    int ex;
    (void)frexp(v, &ex);                 /* v = f * 2^ex, 0.5 <= |f| < 1 */
    const double scale = ldexp(1.0, 8 - ex);
    const double t = v * scale;          /* |t| in [128, 256): 8 significant bits above the point */
    double r = floor(t);
    const double frac = t - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    return r / scale;
}

/* out[i] = bf16?(relu?(y[i])) for the requested steps. */
void oracle_epilogue(const double *y, double *out, int64_t n, int relu, int to_bf16)
{
    for (int64_t i = 0; i < n; ++i) {
        double v = y[i];
        if (relu && v < 0.0) v = 0.0;
        if (to_bf16) v = oracle_round_bf16(v);
        out[i] = v;
    }
}

/* The general convolution with channels-last activations: x (N, [D,] H, W, C)
 * and y (N, [Do,] Ho, Wo, Co), the channel index fastest
 * [PyTorch tensor products and conv2d/conv3d dimension semantics, 6.3];
 * weights stay (Co, C/G, K, K[, K]).  Written with its own indexing, not by
 * transposing into the NCHW function.  bias and S may be NULL. */
int oracle_conv_nhwc(int ndim, const double *x, const double *w, const double *bias, double *y, double *S,
                     int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                     int64_t Co, int64_t K, int64_t s, int64_t p, int64_t d, int64_t G)
{
    gen_geom g;
    if (gen_geom_make(&g, ndim, N, C, D, H, W, Co, K, s, p, d, G) != 0) return -1;
    const int64_t Cg = C / G, Cog = Co / G;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t od = 0; od < g.Do; ++od)
        for (int64_t oh = 0; oh < g.Ho; ++oh)
          for (int64_t ow = 0; ow < g.Wo; ++ow)
            for (int64_t oc = 0; oc < Co; ++oc) {
              const int64_t grp = oc / Cog;
              double acc = 0.0, mag = 0.0;
              for (int64_t kz = 0; kz < g.Kz; ++kz) {
                const int64_t iz = od * g.sz + kz * g.dz - g.pz;
                if (iz < 0 || iz >= g.Dd) continue;
                for (int64_t kh = 0; kh < K; ++kh) {
                  const int64_t iy = oh * s + kh * d - p;
                  if (iy < 0 || iy >= H) continue;
                  for (int64_t kw = 0; kw < K; ++kw) {
                    const int64_t ix = ow * s + kw * d - p;
                    if (ix < 0 || ix >= W) continue;
                    const double *px = x + (((n * g.Dd + iz) * H + iy) * W + ix) * C + grp * Cg;
                    for (int64_t j = 0; j < Cg; ++j) {
                      const double prod = px[j] * w[(((oc * Cg + j) * g.Kz + kz) * K + kh) * K + kw];
                      acc += prod;
                      mag += fabs(prod);
                    }
                  }
                }
              }
              const int64_t o = (((n * g.Do + od) * g.Ho + oh) * g.Wo + ow) * Co + oc;
              y[o] = acc + (bias ? bias[oc] : 0.0);
              if (S) S[o] = mag;
            }
    return 0;
}

/* ---- Winograd F(2x2, 3x3) ---------------------------------------------------
 *
 * [Why use matrix multiplication for convolution, 5.1]: for an r x r kernel
 * and an m x m output block the minimal filtering algorithm uses (m+r-1)^2
 * multiplications instead of m^2 r^2 (F(2x2,3x3): 16 instead of 36), for 3x3
 * kernels, stride 1 and dilation 1 only; it trades multiplications for
 * transform additions and loses accuracy at low precision.  The page names
 * the method but not its matrices; these are the published minimal-filtering
 * ones of F(2,3) (Lavin and Gray, "Fast Algorithms for Convolutional Neural
 * Networks", 2016), nested for two dimensions:
 *     B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1]
 *     G   = [1 0 0; 1/2 1/2 1/2; 1/2 -1/2 1/2; 0 0 1]
 *     A^T = [1 1 1 0; 0 1 -1 -1]
 * Steps for each output channel k and 2x2 output block b (input block d:
 * the 4x4 input patch starting at (2*bh - p, 2*bw - p), zero outside):
 *     U[k][c] = G g[k][c] G^T       (4x4, the transformed 3x3 filter)
 *     V[c][b] = B^T d[c][b] B       (4x4, the transformed input block)
 *     M[k][b] = sum over c of U[k][c] * V[c][b]   (elementwise: 16 products per c)
 *     Y[k][b] = A^T M[k][b] A       (2x2, cropped at the output edge)
 * plus bias.  In fp64 this equals the direct convolution up to rounding (and
 * exactly on integer data, the halves in G being exact).
 * Besides y, Sw holds per output the sum over c and the 16 transform points of
 * |A coefficient| * |U| * |V|: the scale of the error when U and V are rounded
 * to a narrow format before the products.  Sw may be NULL. */
static void wino_mat_4x3_3x4(const double G[4][3], const double g[3][3], double out[4][4])
{
    double t[4][3];
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 3; ++j) {
            t[i][j] = 0.0;
            for (int l = 0; l < 3; ++l) t[i][j] += G[i][l] * g[l][j];
        }
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) {
            out[i][j] = 0.0;
            for (int l = 0; l < 3; ++l) out[i][j] += t[i][l] * G[j][l];
        }
}

int oracle_winograd_f2x2_3x3(const double *x, const double *w, const double *bias, double *y, double *Sw,
                             int64_t N, int64_t C, int64_t H, int64_t W, int64_t Co, int64_t p)
{
    static const double BT[4][4] = {{1, 0, -1, 0}, {0, 1, 1, 0}, {0, -1, 1, 0}, {0, 1, 0, -1}};
    static const double Gm[4][3] = {{1, 0, 0}, {0.5, 0.5, 0.5}, {0.5, -0.5, 0.5}, {0, 0, 1}};
    static const double AT[2][4] = {{1, 1, 1, 0}, {0, 1, -1, -1}};
    const int64_t Ho = oracle_out_dim(H, 3, 1, p), Wo = oracle_out_dim(W, 3, 1, p);
    if (Ho < 0 || Wo < 0 || N < 1 || C < 1 || Co < 1) return -1;
    const int64_t TH = (Ho + 1) / 2, TW = (Wo + 1) / 2;
    /* U for every (k, c) */
    double *U = (double *)malloc(sizeof(double) * 16 * Co * C);
    if (!U) return -1;
    for (int64_t k = 0; k < Co; ++k)
        for (int64_t c = 0; c < C; ++c) {
            double g[3][3], u[4][4];
            for (int i = 0; i < 3; ++i)
                for (int j = 0; j < 3; ++j) g[i][j] = w[((k * C + c) * 3 + i) * 3 + j];
            wino_mat_4x3_3x4(Gm, g, u);
            for (int i = 0; i < 16; ++i) U[(k * C + c) * 16 + i] = u[i / 4][i % 4];
        }
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t bh = 0; bh < TH; ++bh)
        for (int64_t bw = 0; bw < TW; ++bw) {
            /* V for every c of this block */
            double *V = (double *)malloc(sizeof(double) * 16 * C);
            if (!V) continue;
            for (int64_t c = 0; c < C; ++c) {
                double d[4][4], t[4][4];
                for (int i = 0; i < 4; ++i)
                    for (int j = 0; j < 4; ++j) {
                        const int64_t ih = 2 * bh - p + i, iw = 2 * bw - p + j;
                        d[i][j] = (0 <= ih && ih < H && 0 <= iw && iw < W) ? x[((n * C + c) * H + ih) * W + iw] : 0.0;
                    }
                for (int i = 0; i < 4; ++i)          /* t = B^T d */
                    for (int j = 0; j < 4; ++j) {
                        t[i][j] = 0.0;
                        for (int l = 0; l < 4; ++l) t[i][j] += BT[i][l] * d[l][j];
                    }
                for (int i = 0; i < 4; ++i)          /* V = t B */
                    for (int j = 0; j < 4; ++j) {
                        double v = 0.0;
                        for (int l = 0; l < 4; ++l) v += t[i][l] * BT[j][l];
                        V[c * 16 + i * 4 + j] = v;
                    }
            }
            for (int64_t k = 0; k < Co; ++k) {
                double M[16], Ma[16];
                for (int i = 0; i < 16; ++i) { M[i] = 0.0; Ma[i] = 0.0; }
                for (int64_t c = 0; c < C; ++c)
                    for (int i = 0; i < 16; ++i) {
                        const double uv = U[(k * C + c) * 16 + i] * V[c * 16 + i];
                        M[i] += uv;
                        Ma[i] += fabs(uv);
                    }
                for (int a = 0; a < 2; ++a)
                    for (int b = 0; b < 2; ++b) {
                        const int64_t oh = 2 * bh + a, ow = 2 * bw + b;
                        if (oh >= Ho || ow >= Wo) continue;
                        double acc = 0.0, mag = 0.0;  /* (A^T M A)[a][b] */
                        for (int i = 0; i < 4; ++i)
                            for (int j = 0; j < 4; ++j) {
                                acc += AT[a][i] * M[i * 4 + j] * AT[b][j];
                                mag += fabs(AT[a][i] * AT[b][j]) * Ma[i * 4 + j];
                            }
                        const int64_t o = ((n * Co + k) * Ho + oh) * Wo + ow;
                        y[o] = acc + (bias ? bias[k] : 0.0);
                        if (Sw) Sw[o] = mag;
                    }
            }
            free(V);
        }
    free(U);
    return 0;
}

/* Threads the OpenMP runtime will use (1 when built without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
