// conv_internal.h -- shapes and kernel launchers shared inside libconvfwd.so.
// Not part of the public ABI (that is include/conv_fwd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "conv_fwd.h"

namespace convfwd {

// One convolution problem.  2D problems are carried as 3D with D = Do = 1,
// Kd = 1, pad_d = 0, stride_d = 1, dil_d = 1, so every kernel indexes (d, h, w).
// Tap (kd, kh, kw) of output (od, oh, ow) reads input
// (od*sd + kd*dild - pd, oh*s + kh*dil - p, ow*s + kw*dil - p); output channel
// oc belongs to group oc / (Co/G) and reads the C/G input channels of that group.
struct Shape {
    int ndim;               // 2 or 3
    int N, C, D, H, W;      // input  N x C x D x H x W
    int Co;                 // output channels
    int K, s, p;            // square/cubic kernel, one stride, one symmetric pad
    int Kd, sd, pd;         // depth kernel/stride/pad: (K, s, p) in 3D, (1, 1, 0) in 2D
    int Do, Ho, Wo;         // output spatial extents (Do = 1 in 2D)
    int dil = 1, dild = 1;  // dilation in H/W and in depth (dild = 1 in 2D)
    int G = 1;              // groups: divides C and Co
    int ups = 1, upsd = 1;  // zero insertion of the input (data gradient of a strided
                            // convolution; only the general kernel's upsampled mode reads these)
    int out_bf16 = 0;       // y holds bf16 bits (fp32 result rounded to nearest even), not fp32
    int relu = 0;           // y = max(y, 0) before the store
    int nhwc = 0;           // x and y channels-last: (N, [D,] H, W, C); w stays (Co, C/G, taps)

    __host__ __device__ int Cg() const { return C / G; }                                // input channels per group
    __host__ __device__ int Cog() const { return Co / G; }                              // output channels per group
    __host__ __device__ bool plain() const { return dil == 1 && G == 1; }
    __host__ __device__ bool plain_io() const { return !out_bf16 && !relu && !nhwc; }
    __host__ __device__ int64_t taps() const { return (int64_t)Kd * K * K; }            // K^ndim
    __host__ __device__ int64_t kgemm() const { return (int64_t)Cg() * taps(); }       // reduction per group
    __host__ __device__ int64_t xcol_rows() const { return (int64_t)C * taps(); }      // rows of X_col
    __host__ __device__ int64_t in_plane() const { return (int64_t)D * H * W; }
    __host__ __device__ int64_t out_plane() const { return (int64_t)Do * Ho * Wo; }
    __host__ __device__ int64_t pixels() const { return (int64_t)N * out_plane(); }    // GEMM N dimension
    __host__ __device__ int64_t x_elems() const { return (int64_t)N * C * in_plane(); }
    __host__ __device__ int64_t w_elems() const { return (int64_t)Co * kgemm(); }
    __host__ __device__ int64_t y_elems() const { return (int64_t)Co * pixels(); }
    __host__ __device__ int64_t xcol_elems() const { return xcol_rows() * pixels(); }
};

// Kernel launchers.  Each enqueues on `st` and returns hipGetLastError().
hipError_t launch_im2col_bf16(const Shape &sh, const uint16_t *x, uint16_t *xcol, hipStream_t st);
// the explicit GEMM with direct-to-LDS loads in a ring of stage buffers (k_xcol_gemm.hip)
bool gemm_xcol_dma_supported(const Shape &sh, const void *xcol, const void *w);
hipError_t launch_gemm_xcol_dma_bf16(const Shape &sh, const uint16_t *w, const uint16_t *xcol, const float *bias,
                                     float *y, hipStream_t st);
hipError_t launch_gemm_xcol_bf16(const Shape &sh, const uint16_t *w, const uint16_t *xcol,
                                 const float *bias, float *y, hipStream_t st);
hipError_t launch_igemm_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w,
                             const float *bias, float *y, hipStream_t st, void *ws = nullptr,
                             size_t ws_bytes = 0);
// Workspace bytes the MFMA route can use for this shape (0: none).
size_t igemm_workspace_bytes(const Shape &sh, const void *x, const void *w);
// The MFMA route with weights already packed into ws by launch_pack_w3x3
// (only for shapes where igemm_workspace_bytes() > 0).
hipError_t launch_igemm_prepacked_bf16(const Shape &sh, const uint16_t *x, const uint16_t *wpack,
                                       const float *bias, float *y, hipStream_t st);
hipError_t launch_valu_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w,
                            const float *bias, float *y, hipStream_t st);
// Route-specific launchers behind the two dispatchers above.
hipError_t launch_igemm_generic_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w,
                                     const float *bias, float *y, hipStream_t st);
// The general kernel over x seen through zero insertion: a virtual coordinate
// v of the (D-1)*upsd+1 x (H-1)*ups+1 x (W-1)*ups+1 input reads x[v/ups] when
// ups divides v, else 0.  sh.Do/Ho/Wo are set by the caller.
hipError_t launch_igemm_upsampled_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias,
                                       float *y, hipStream_t st);
// Backward pieces (k_bwd.hip).  wflip: w (Co, C/G, taps) -> (C, Co/G, taps)
// with the taps reversed, the weight of the data gradient as a convolution.
void launch_flip_weights_bf16(const Shape &sh, const uint16_t *w, uint16_t *wflip, hipStream_t st);
// Weight gradient: partial sums over `splits` pixel ranges into part
// (splits x Co x C/G*taps fp32), then their fixed-order sum into dw.
int wgrad_splits(const Shape &sh, bool aligned);      // aligned: x and dout 16-byte aligned
int64_t wgrad_workspace_floats(const Shape &sh);        // enough for either alignment
hipError_t launch_wgrad_bf16(const Shape &sh, const uint16_t *x, const uint16_t *dout, float *part, float *dw,
                             float *db, hipStream_t st);   // db: NULL or the bias gradient, computed too
// Winograd F(2x2, 3x3): 2D, K=3, stride 1, dilation 1, groups 1, NCHW, C % 16 == 0.
bool winograd_supported(const Shape &sh);
size_t winograd_workspace_bytes(const Shape &sh);
// ws: 256-byte aligned, winograd_workspace_bytes(sh) bytes (transformed weights and inputs).
hipError_t launch_winograd_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias, float *y,
                                void *ws, hipStream_t st);
// db[oc] = sum of dout over images and positions (fixed order).
// db from dout; part holds (ranges x C_out) floats and may be the front of
// the weight-gradient workspace
int bias_grad_ranges(const Shape &sh);
hipError_t launch_bias_grad_bf16(const Shape &sh, const uint16_t *dout, float *part, float *db, hipStream_t st);
bool conv3x3s1_supported(const Shape &sh, const void *x, const void *w);
// Workspace for the repacked weights of the 3x3 kernel (bytes).
size_t conv3x3s1_workspace_bytes(const Shape &sh);
// wpack: NULL (weights transposed in the kernel) or a 16-byte aligned buffer of
// conv3x3s1_workspace_bytes() bytes that receives the repacked weights first
// (prepacked: it already holds them; w is then not read).
hipError_t launch_conv3x3s1_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, uint16_t *wpack,
                                 const float *bias, float *y, hipStream_t st, bool prepacked = false);
// Repack OIHW 3x3 weights (C % 16 == 0, Co % 128 == 0) into the per-stage LDS
// images both 3x3 kernels load: Co*C*9*2 bytes at wpack.
void launch_pack_w3x3(const Shape &sh, const uint16_t *w, uint16_t *wpack, hipStream_t st);
// Column-group 3x3 stride-1 kernel (packed weights only).
bool conv3x3cg_supported(const Shape &sh, const void *x, const void *w);
// persistent variant of the column-group kernel (NCHW, dilation 1, groups 1),
// and whether to prefer it over one workgroup per tile for this shape
bool conv3x3cgp_supported(const Shape &sh, const void *x, const void *w);
bool conv3x3cgp_preferred(const Shape &sh);
hipError_t launch_conv3x3cgp_bf16(const Shape &sh, const uint16_t *x, const uint16_t *wpack, const float *bias,
                                  float *y, hipStream_t st);
hipError_t launch_conv3x3cg_bf16(const Shape &sh, const uint16_t *x, const uint16_t *wpack, const float *bias,
                                 float *y, hipStream_t st);
// Pointwise (K = 1, stride 1, pad 0) GEMM kernel.
bool conv1x1_supported(const Shape &sh, const void *x, const void *w);
hipError_t launch_conv1x1_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w,
                               const float *bias, float *y, hipStream_t st);
// Short-reduction (C_in * K^dims <= 128) implicit GEMM: stems and first 3D layers.
bool smallk_supported(const Shape &sh);
hipError_t launch_smallk_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias,
                              float *y, hipStream_t st);
hipError_t launch_valu_generic_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w,
                                    const float *bias, float *y, hipStream_t st);
hipError_t launch_valu_f32(const Shape &sh, const float *x, const float *w,
                           const float *bias, float *y, hipStream_t st);
// Depthwise-style kernel for one input channel per group (C/G == 1), 2D.
bool depthwise_supported(const Shape &sh);
hipError_t launch_depthwise_bf16(const Shape &sh, const uint16_t *x, const uint16_t *w, const float *bias,
                                 float *y, hipStream_t st);
hipError_t launch_depthwise_f32(const Shape &sh, const float *x, const float *w, const float *bias,
                                float *y, hipStream_t st);

// The library's own device scratch array (static_scratch.hip): its size, and
// its address on the current device (looked up once per device, then kept).
constexpr size_t kStaticScratchBytes = CONV_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(void **ptr);

}  // namespace convfwd
