/*
 * conv_fwd.h -- C ABI of libconvfwd.so, a convolution forward engine for one
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  For a 2D convolution with one square kernel size K, one
 * stride s and one symmetric zero pad p (page "Hand-writing Conv2D", 1.1-1.2):
 *
 *     y[n][oc][oh][ow] = bias[oc] + sum_{ic, kh, kw}
 *                        x[n][ic][oh*s + kh - p][ow*s + kw - p] * w[oc][ic][kh][kw]
 *
 * where a tap whose input coordinate falls outside the input contributes 0
 * (zero padding by bounds checks, no padded copy).  The output size per
 * spatial dimension is  out = floor((in + 2p - K)/s) + 1  (same section).
 * The engine evaluates it as the product  W_row (C_out x C_in*K*K) @ X_col
 * (C_in*K*K x N*H_out*W_out)  of the page "Why use matrix multiplication for
 * convolution", 2.2-2.3, either with X_col materialised in device memory
 * (the *_explicit and *_im2col entry points) or gathered tile by tile inside
 * the GEMM kernel and never stored (implicit GEMM, same page, 4.3).  The 3D
 * form adds a depth dimension with the same K, s, p (page "PyTorch tensor
 * products and conv2d/conv3d dimension semantics", 5.1-5.2).
 *
 * Conventions for every entry point below:
 *   Layout     x is dense NCHW (2D) or NCDHW (3D); w is dense OIHW / OIDHW,
 *              i.e. (C_out, C_in, K, K[, K]); bias is (C_out); y is dense
 *              N C_out H_out W_out (or N C_out D_out H_out W_out).  Strided
 *              views are not accepted: pass contiguous buffers.
 *   Types      "bf16" pointers hold raw bfloat16 bit patterns (uint16_t).
 *              The output is always fp32; accumulation is fp32; bias is fp32.
 *   Memory     every tensor pointer is a DEVICE pointer owned by the caller.
 *              The library allocates nothing, frees nothing and keeps no
 *              pointer after the call returns (conv2d_fwd_bf16_noalloc uses
 *              a fixed array of its own instead of a workspace; see there).
 *   Streams    `stream` is a hipStream_t (NULL = the null stream).  Work is
 *              enqueued on it and the call returns before the work finishes;
 *              the caller synchronises.  Calls on one stream run in order.
 *   Errors     arguments are validated on the host BEFORE any HIP call; on a
 *              validation error nothing is launched and y is not written.  A
 *              status other than CONV_OK is returned, never an exit or abort.
 *              CONV_ERR_HIP reports a failed launch (the HIP error is then
 *              also left in the runtime's last-error slot).
 *   Limits     each tensor (x, w, y, X_col) must hold fewer than 2^31
 *              elements; N, C_in, C_out, spatial sizes and K >= 1; stride >= 1;
 *              pad >= 0; every padded input extent must be >= K.
 *   Aliasing   y must not overlap x, w, bias (or the workspace).
 */
#ifndef CONV_FWD_H
#define CONV_FWD_H

#include <stddef.h>
#include <stdint.h>

/* Only the functions below are exported from the shared library. */
#define CONV_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONV_OK = 0,
    CONV_ERR_NULL = 1,       /* a required pointer (x, w, y, workspace) is NULL            */
    CONV_ERR_PARAM = 2,      /* a size < 1, K < 1, stride < 1, pad < 0 (or, for the general
                                entry points, dilation < 1 or groups not dividing C_in, C_out) */
    CONV_ERR_SHAPE = 3,      /* in + 2*pad < K in some spatial dimension (no output)        */
    CONV_ERR_OVERFLOW = 4,   /* a tensor would hold 2^31 or more elements                   */
    CONV_ERR_ALIAS = 5,      /* y overlaps x, w, bias or the workspace                      */
    CONV_ERR_WORKSPACE = 6,  /* workspace smaller than conv*_im2col_bytes() requires        */
    CONV_ERR_ALGO = 7,       /* the requested algorithm does not exist for this dtype/shape */
    CONV_ERR_HIP = 8,        /* a HIP launch failed                                         */
    CONV_ERR_SCRATCH = 9     /* conv2d_fwd_bf16_noalloc: the problem needs more than
                                CONV_STATIC_SCRATCH_BYTES of scratch                        */
} conv_status_t;

/* Kernel route.  AUTO picks by shape, for bf16: first the matrix cores'
 * short-reduction kernel when C_in/groups*K^dims <= 128 and one output row's
 * input patch fits its LDS tile (this takes the thin stem layer, 3 channels x
 * 3x3, and the 3-channel 3D layer); else one input channel per group in 2D
 * (depthwise) -> the VALU depthwise kernel; else a reduction of at most 32
 * (C_in/groups*K^dims) -> the VALU direct kernel; else the MFMA implicit
 * GEMM.  fp32 -> VALU.  MFMA is bf16-only (CONV_ERR_ALGO for fp32).
 * CONV_ALGO_VALU forces the direct FMA route for any bf16 shape. */
typedef enum {
    CONV_ALGO_AUTO = 0,
    CONV_ALGO_MFMA = 1,      /* implicit GEMM on bf16 matrix cores, fp32 accumulate */
    CONV_ALGO_VALU = 2,      /* direct convolution, fp32 FMA on the vector ALUs       */
    CONV_ALGO_WINOGRAD = 3   /* Winograd F(2x2,3x3) ("Why use matrix multiplication for
                                convolution", 5.1): conv_fwd_ex_bf16 only, with a
                                workspace; 3x3, stride 1, dilation 1, groups 1, NCHW,
                                C_in % 16 == 0.  Never chosen by AUTO.  The transformed
                                operands are fp16: x and w are first scaled by powers of
                                two chosen from max|x| and max|w| (one pass over both), so
                                any finite bf16 data fits; elements more than ~2^27 below
                                their tensor's largest magnitude lose precision (fp16
                                subnormals), which the 1e-3 * sum|x w| bound absorbs. */
} conv_algo_t;

/* floor((in + 2*pad - K)/stride) + 1, or -1 if in < 1, K < 1, stride < 1,
 * pad < 0 or in + 2*pad < K ("Hand-writing Conv2D", 1.1; the explicit reject
 * of a negative numerator follows "Conv2d from the official docs", 3.2, which
 * warns that C division truncates rather than floors for negatives). */
CONV_API int64_t conv_out_dim(int64_t in, int64_t K, int64_t stride, int64_t pad);

/* Static, NUL-terminated text for a status code; never NULL. */
CONV_API const char *conv_status_str(int status);

/* Library version as major*10000 + minor*100 + patch. */
CONV_API int conv_version(void);

/* ---- direct entry points: y = conv(x, w) + bias ------------------------- */

/* 2D, bf16 inputs and weights, fp32 bias (NULL = no bias) and output.
 * Shapes: x (N, C_in, H, W), w (C_out, C_in, K, K), y (N, C_out, H_out, W_out). */
CONV_API conv_status_t conv2d_fwd_bf16(const uint16_t *x, const uint16_t *w, const float *bias, float *y,
                              int N, int C_in, int H, int W, int C_out,
                              int K, int stride, int pad, int algo, void *stream);

/* 2D, fp32 everywhere (VALU route only).  Same shapes. */
CONV_API conv_status_t conv2d_fwd_f32(const float *x, const float *w, const float *bias, float *y,
                             int N, int C_in, int H, int W, int C_out,
                             int K, int stride, int pad, int algo, void *stream);

/* 3D, bf16 inputs: x (N, C_in, D, H, W), w (C_out, C_in, K, K, K),
 * y (N, C_out, D_out, H_out, W_out). */
CONV_API conv_status_t conv3d_fwd_bf16(const uint16_t *x, const uint16_t *w, const float *bias, float *y,
                              int N, int C_in, int D, int H, int W, int C_out,
                              int K, int stride, int pad, int algo, void *stream);

/* 3D, fp32 everywhere (VALU route only). */
CONV_API conv_status_t conv3d_fwd_f32(const float *x, const float *w, const float *bias, float *y,
                             int N, int C_in, int D, int H, int W, int C_out,
                             int K, int stride, int pad, int algo, void *stream);

/* ---- with a workspace --------------------------------------------------- */

/* Bytes of device workspace conv2d_fwd_bf16_ws can use for these arguments:
 * the 3x3 stride-1 pad-1 MFMA kernels (C_in % 16 == 0, C_out % 128 == 0,
 * W % 8 == 0, and 32 <= W <= 64, or C_in >= 32 and 8 <= W <= 64) repack the
 * weights once per call into C_out*C_in*9*2 bytes laid out as per-stage LDS
 * images, so that they stream them with coalesced direct-to-LDS loads
 * instead of transposing OIHW in every workgroup.  0 when no route uses a
 * workspace. */
CONV_API size_t conv2d_fwd_workspace_bytes(int N, int C_in, int H, int W, int C_out,
                                           int K, int stride, int pad, int algo);

/* conv2d_fwd_bf16 plus a caller-owned device workspace (16-byte aligned, at
 * least conv2d_fwd_workspace_bytes() bytes; may be NULL when that is 0).  The
 * workspace is overwritten; the result equals conv2d_fwd_bf16's.  Returns
 * CONV_ERR_WORKSPACE if it is needed and missing, too small or misaligned,
 * CONV_ERR_ALIAS if it overlaps x, w or y.  Two calls in flight at once must
 * not share a workspace. */
CONV_API conv_status_t conv2d_fwd_bf16_ws(const uint16_t *x, const uint16_t *w, const float *bias,
                                          float *y, void *workspace, size_t workspace_bytes,
                                          int N, int C_in, int H, int W, int C_out,
                                          int K, int stride, int pad, int algo, void *stream);

/* The two halves of conv2d_fwd_bf16_ws, for callers whose weights do not
 * change between calls (the weight view W_row of "Why use matrix
 * multiplication for convolution", 2.2, prepared once): */

/* Writes the packed weights for these arguments into the workspace (16-byte
 * aligned, >= conv2d_fwd_workspace_bytes() bytes) on `stream`.  w: OIHW bf16,
 * 16-byte aligned.  Returns CONV_ERR_ALGO when no route of these arguments
 * uses packed weights (conv2d_fwd_workspace_bytes() == 0) or w is not 16-byte
 * aligned, CONV_ERR_WORKSPACE if the workspace is too small or misaligned,
 * CONV_ERR_ALIAS if it overlaps w. */
CONV_API conv_status_t conv2d_pack_weights_bf16(const uint16_t *w, void *workspace, size_t workspace_bytes,
                                                int N, int C_in, int H, int W, int C_out,
                                                int K, int stride, int pad, int algo, void *stream);

/* conv2d_fwd_bf16 with the weights taken from a workspace that
 * conv2d_pack_weights_bf16 filled for the same sizes and algo (the weight
 * tensor itself is not read).  Same result as conv2d_fwd_bf16_ws.  The
 * workspace is only read, so concurrent calls may share it.  Errors as
 * conv2d_fwd_bf16_ws, plus CONV_ERR_ALGO when these arguments have no
 * packed-weight route. */
CONV_API conv_status_t conv2d_fwd_bf16_prepacked(const uint16_t *x, const void *workspace,
                                                 size_t workspace_bytes, const float *bias, float *y,
                                                 int N, int C_in, int H, int W, int C_out,
                                                 int K, int stride, int pad, int algo, void *stream);

/* ---- without allocation ------------------------------------------------- */

/* Size of the library's own device scratch array (one per GPU, kept until
 * the process ends), used by conv2d_fwd_bf16_noalloc. */
#define CONV_STATIC_SCRATCH_BYTES ((size_t)8 << 20)

/* For callers that cannot allocate device memory (code under stream or graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and result as conv2d_fwd_bf16_ws, with the workspace taken from
 * a file-scope device array of CONV_STATIC_SCRATCH_BYTES inside the library
 * instead of from the caller.  No hipMalloc, hipFree or other allocating call
 * is made.  The array's address on the current device is looked up on the
 * first call on that device.  Arguments, layouts, ownership and errors as
 * conv2d_fwd_bf16_ws (minus the workspace pair), plus CONV_ERR_SCRATCH, before
 * any launch, when conv2d_fwd_workspace_bytes() of these arguments exceeds
 * CONV_STATIC_SCRATCH_BYTES (3x3 layers with C_out*C_in*9*2 > 8 MiB, e.g.
 * C_in = C_out = 1024), and CONV_ERR_HIP if the address lookup fails.  All
 * calls on one GPU share its one array and every call overwrites it (nothing
 * in it needs to start at zero): two calls that can run at the same time on
 * one GPU (different streams, or different host threads) race and may give
 * wrong results; serialise them, e.g. on one stream. */
CONV_API conv_status_t conv2d_fwd_bf16_noalloc(const uint16_t *x, const uint16_t *w, const float *bias,
                                               float *y, int N, int C_in, int H, int W, int C_out,
                                               int K, int stride, int pad, int algo, void *stream);

/* ---- explicit im2col path ("Why use matrix multiplication for convolution",
 *      2.2 and 3.1): X_col is materialised in caller-owned device memory. ---- */

/* Bytes of the bf16 X_col matrix, (C_in*K*K) x (N*H_out*W_out) elements, for
 * these arguments; 0 if the arguments are invalid or X_col would hold 2^31 or
 * more elements.  D = 1 and the 2D formula apply when ndim == 2. */
CONV_API size_t conv_im2col_bytes(int ndim, int N, int C_in, int D, int H, int W,
                         int K, int stride, int pad);

/* X_col[r][j] = x[n][ic][oh*s+kh-p][ow*s+kw-p] (0 outside the input), with
 * row r = (ic*K + kh)*K + kw and column j = (n*H_out + oh)*W_out + ow, stored
 * row-major as bf16 into xcol (which must hold conv_im2col_bytes() bytes).
 * The copy is exact (bit for bit). */
CONV_API conv_status_t conv2d_im2col_bf16(const uint16_t *x, uint16_t *xcol,
                                 int N, int C_in, int H, int W,
                                 int K, int stride, int pad, void *stream);

/* 3D twin: row r = ((ic*K + kd)*K + kh)*K + kw, column
 * j = ((n*D_out + od)*H_out + oh)*W_out + ow. */
CONV_API conv_status_t conv3d_im2col_bf16(const uint16_t *x, uint16_t *xcol,
                                 int N, int C_in, int D, int H, int W,
                                 int K, int stride, int pad, void *stream);

/* im2col into `workspace`, then one MFMA GEMM  W_row @ X_col  whose epilogue
 * adds bias and writes y directly in N C_out H_out W_out order (the reshape and
 * axis swap of "Why use matrix multiplication for convolution", 3.2, fused
 * into the store).  workspace: device memory of at least
 * conv_im2col_bytes(2, ...) bytes, owned by the caller, clobbered. */
CONV_API conv_status_t conv2d_fwd_bf16_explicit(const uint16_t *x, const uint16_t *w, const float *bias,
                                       float *y, void *workspace, size_t workspace_bytes,
                                       int N, int C_in, int H, int W, int C_out,
                                       int K, int stride, int pad, void *stream);

/* 3D twin of conv2d_fwd_bf16_explicit; workspace of conv_im2col_bytes(3, ...). */
CONV_API conv_status_t conv3d_fwd_bf16_explicit(const uint16_t *x, const uint16_t *w, const float *bias,
                                       float *y, void *workspace, size_t workspace_bytes,
                                       int N, int C_in, int D, int H, int W, int C_out,
                                       int K, int stride, int pad, void *stream);

/* ---- general problems: dilation and groups -------------------------------
 *
 * Dilation d places the K taps of a window d inputs apart, so a window spans
 * d(K-1)+1 inputs and  out = floor((in + 2*pad - d(K-1) - 1)/stride) + 1
 * ("PyTorch tensor products and conv2d/conv3d dimension semantics", 4.2;
 * "Conv2d from the official docs", 3.2-3.3).  Groups G cut C_in and C_out into
 * G equal consecutive blocks; output block g reads input block g only, and the
 * weight holds C_in/G input channels per filter (same pages, 4.3 and 3.4).
 * G == C_in is the depthwise layer.  With g = oc / (C_out/G):
 *
 *     y[n][oc][oh][ow] = bias[oc] + sum_{j < C_in/G, kh, kw}
 *         x[n][g*C_in/G + j][oh*s + kh*d - p][ow*s + kw*d - p] * w[oc][j][kh][kw]
 *
 * (3D adds od*s + kd*d - p on the depth axis).  Taps outside the input add 0.
 * Layouts as above, except w is (C_out, C_in/G, K, K[, K]).  With d = 1 and
 * G = 1 every entry point below computes exactly what its conv2d_/conv3d_
 * counterpart computes.  Extra errors: CONV_ERR_PARAM when dilation < 1,
 * groups < 1, groups does not divide C_in and C_out, or ndim is not 2 or 3;
 * CONV_ERR_NULL when the parameter block is NULL. */
typedef struct {
    int ndim;        /* 2 or 3                                                  */
    int N, C_in;
    int D;           /* input depth; ignored (taken as 1) when ndim == 2         */
    int H, W;
    int C_out;
    int K;           /* kernel extent, the same in every spatial dimension       */
    int stride, pad; /* the same in every spatial dimension                      */
    int dilation;    /* >= 1                                                     */
    int groups;      /* >= 1, divides C_in and C_out                             */
} conv_params_t;

/* floor((in + 2*pad - dilation*(K-1) - 1)/stride) + 1, or -1 on a bad
 * parameter or when the dilated window does not fit in the padded input. */
CONV_API int64_t conv_out_dim_dilated(int64_t in, int64_t K, int64_t stride, int64_t pad, int64_t dilation);

/* y = conv(x, w) + bias for a general problem, bf16 x and w, fp32 bias (NULL =
 * none) and y.  AUTO: one input channel per group (C_in/G == 1, 2D) -> the
 * depthwise VALU kernel, which reads each input once and writes each output
 * once; a per-group reduction (C_in/G * K^ndim) <= 32 -> the direct VALU
 * kernel; otherwise the MFMA implicit GEMM, one GEMM of C_out/G x
 * (C_in/G * K^ndim) per group.  It takes no workspace: the 3x3 kernels that
 * read packed weights (dilation 1 or 2 with pad = dilation, or groups of 32
 * output channels) are reached through conv_fwd_ex_bf16 with a workspace. */
CONV_API conv_status_t conv_fwd_bf16(const conv_params_t *params, const uint16_t *x, const uint16_t *w,
                                     const float *bias, float *y, int algo, void *stream);

/* fp32 twin (VALU route only). */
CONV_API conv_status_t conv_fwd_f32(const conv_params_t *params, const float *x, const float *w,
                                    const float *bias, float *y, int algo, void *stream);

/* Bytes of the bf16 X_col of a general problem: C_in*K^ndim rows (groups do
 * not change X_col; group g uses rows [g, g+1) * C_in/G * K^ndim) by
 * N * (output positions) columns; 0 on invalid parameters or when X_col would
 * hold 2^31 or more elements. */
CONV_API size_t conv_xcol_bytes(const conv_params_t *params);

/* X_col of a general problem: row ((ic*K + kd)*K + kh)*K + kw (kd absent in
 * 2D), column in output order, entry x at the dilated tap coordinate, 0
 * outside.  xcol must hold conv_xcol_bytes() bytes.  Exact copy. */
CONV_API conv_status_t conv_im2col_bf16(const conv_params_t *params, const uint16_t *x, uint16_t *xcol,
                                        void *stream);

/* conv_im2col_bf16 into the workspace (>= conv_xcol_bytes() bytes), then per
 * group g the GEMM W_row[g] (C_out/G x C_in/G*K^ndim) @ X_col[rows of g] with
 * bias, stored into y in N C_out (D) H W order. */
CONV_API conv_status_t conv_fwd_explicit_bf16(const conv_params_t *params, const uint16_t *x,
                                              const uint16_t *w, const float *bias, float *y,
                                              void *workspace, size_t workspace_bytes, void *stream);

/* ---- options: channels-last layout, ReLU, bf16 output ---------------------
 *
 * layout CONV_LAYOUT_NHWC: x is (N, [D,] H, W, C_in) and y is (N, [D_out,]
 * H_out, W_out, C_out), the channel index fastest (channels_last, "PyTorch
 * tensor products and conv2d/conv3d dimension semantics", 6.3); w stays
 * (C_out, C_in/G, K, K[, K]).  relu = 1: y = max(y, 0) after the bias (the
 * activation that follows the convolution in the same page, 6.2).
 * out_dtype CONV_OUT_BF16: y holds bf16 bits, the fp32 result rounded to the
 * nearest bf16, ties to even; accumulation stays fp32.  A NULL options
 * pointer means NCHW, fp32, no ReLU. */
typedef enum { CONV_LAYOUT_NCHW = 0, CONV_LAYOUT_NHWC = 1 } conv_layout_t;
typedef enum { CONV_OUT_F32 = 0, CONV_OUT_BF16 = 1 } conv_out_t;
typedef struct {
    int layout;      /* conv_layout_t, for x and y                  */
    int out_dtype;   /* conv_out_t                                   */
    int relu;        /* 0 or 1                                       */
} conv_options_t;

/* Workspace conv_fwd_ex_bf16 can use (C_out x C_in/G x 9 bf16: the packed
 * weights of the 3x3 column-group kernels, for 3x3 stride-1 layers with
 * dilation 1 or 2 and pad = dilation, or with groups of 32 output channels
 * (NCHW, dilation 1); any epilogue, and channels-last for groups 1) or, with
 * algo CONV_ALGO_WINOGRAD, needs
 * (the fp16 transformed weights, 16 x C_out x C_in, and transformed input
 * blocks, 16 x N*ceil(H_out/2)*ceil(W_out/2) x C_in rounded up to a multiple
 * of 32); 0 when none, or on
 * invalid arguments or a shape Winograd does not take. */
CONV_API size_t conv_fwd_ex_workspace_bytes(const conv_params_t *params, const conv_options_t *opts, int algo);

/* conv_fwd_bf16 with options.  y is float* (fp32) or uint16_t* (bf16 bits)
 * as out_dtype says.  workspace: NULL, or 16-byte aligned (256-byte aligned
 * with Winograd) device memory of at least conv_fwd_ex_workspace_bytes()
 * bytes (overwritten).  Kernels that
 * do not take an option step aside for the general ones: channels-last runs
 * on the 3x3 column-group kernel (groups 1), a channels-last pointwise
 * kernel, and otherwise the general implicit GEMM and the direct VALU kernel;
 * the 3x3, pointwise and depthwise kernels apply ReLU and bf16 output in
 * their own epilogue.
 * algo CONV_ALGO_WINOGRAD computes U = G g G^T and V = B^T d B in fp16, the
 * 16 transform-point GEMMs on the matrix cores with fp32 accumulation, and
 * A^T M A per 2x2 block; its error scale is the transform-domain magnitude
 * sum, up to ~4x the direct one on N(0,1) data (the page's low-precision
 * caveat).  Extra errors: CONV_ERR_PARAM for an unknown layout, out_dtype or
 * relu value; CONV_ERR_WORKSPACE as for conv2d_fwd_bf16_ws (required with
 * Winograd); CONV_ERR_ALGO when Winograd does not take the shape. */
CONV_API conv_status_t conv_fwd_ex_bf16(const conv_params_t *params, const conv_options_t *opts, const uint16_t *x,
                                        const uint16_t *w, const float *bias, void *y, void *workspace,
                                        size_t workspace_bytes, int algo, void *stream);

/* fp32 twin (VALU route). */
CONV_API conv_status_t conv_fwd_ex_f32(const conv_params_t *params, const conv_options_t *opts, const float *x,
                                       const float *w, const float *bias, void *y, int algo, void *stream);

/* ---- backward: gradients of y = conv(x, w) + b ----------------------------
 *
 * With upstream gradient dout (the shape of y) ("Hand-writing Conv2D", 5.1;
 * "Why use matrix multiplication for convolution", 3.3):
 *     db[oc]             = sum over n and output positions of dout[n][oc]
 *     dw[oc][j][taps]    = sum over n, output positions of dout[n][oc][o] *
 *                          x[n][g*C_in/G + j][o*s + k*d - p]   (dW_row = dout_col @ X_col^T)
 *     dx[n][ic][i]       = sum over the (oc, o, k) whose tap k of output o read
 *                          input i of w[oc][j][k] * dout[n][oc][o]  (col2im(W_row^T @ dout_col))
 * for the general problem of conv_params_t (dilation, groups, 2D/3D).  x, w and
 * dout are bf16 bits; dx, dw, db are fp32; accumulation is fp32.  Results are
 * bitwise reproducible (fixed summation order, no atomics).  Errors as for
 * conv_fwd_bf16, plus CONV_ERR_WORKSPACE when the workspace is missing, too
 * small or not 16-byte aligned, and CONV_ERR_ALIAS when an output overlaps an
 * input or the workspace. */

/* Device workspace for conv_bwd_data_bf16: the flipped weights (and, for 3x3
 * stride-1 layers, their per-stage packing); 0 on invalid parameters. */
CONV_API size_t conv_bwd_data_workspace_bytes(const conv_params_t *params);

/* dx (N, C_in, [D,] H, W) from dout and w.  The data gradient is computed as
 * a forward convolution of dout with w transposed per group (C_in x C_out/G)
 * and every tap reversed, pad d(K-1) - p, on the forward kernels; a strided
 * layer reads dout through zero insertion (the transposed convolution) on the
 * general implicit-GEMM kernel.  The workspace is overwritten. */
CONV_API conv_status_t conv_bwd_data_bf16(const conv_params_t *params, const uint16_t *dout, const uint16_t *w,
                                          float *dx, void *workspace, size_t workspace_bytes, void *stream);

/* Device workspace for conv_bwd_weight_bf16: fp32 partial sums of dw (and
 * of db) over ranges of output positions; 0 on invalid parameters. */
CONV_API size_t conv_bwd_weight_workspace_bytes(const conv_params_t *params);

/* dw (C_out, C_in/G, K, K[, K]) and, when db is not NULL, db (C_out) from x
 * and dout.  dw is reduced over output positions in ranges on the matrix
 * cores, then the ranges are added in a fixed order.  The workspace is
 * overwritten. */
CONV_API conv_status_t conv_bwd_weight_bf16(const conv_params_t *params, const uint16_t *x, const uint16_t *dout,
                                            float *dw, float *db, void *workspace, size_t workspace_bytes,
                                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CONV_FWD_H */
