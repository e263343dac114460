// mfma_common.h -- small device helpers for the bf16 matrix-core kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfwd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16_bf16: D(32x32) += A(32x16) * B(16x32), fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32]; it
// receives D[8*(i/4) + 4*(l/32) + i%4][l%32] in accumulator slot i.
__device__ __forceinline__ f32x16_t mfma32x32x16(const uint4 &a, const uint4 &b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in slot i by lane l.
__device__ __forceinline__ int mfma32_row(int i, int lane) {
    return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ uint4 pack8(const uint16_t (&v)[8]) {
    uint4 r;
    r.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
    r.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
    r.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
    r.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
    return r;
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at p (raw buffer, 32-bit offsets).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr uint32_t kOob = 0x80000000u;     // buffer offset past any valid byte: loads 0, stores dropped

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The output epilogue of every kernel: optional ReLU, then an fp32 store or a
// bf16 store (y then holds uint16 bits) at element index i.
__device__ __forceinline__ void store_out(float *y, int64_t i, float v, int out_bf16, int relu) {
    if (relu) v = fmaxf(v, 0.f);
    if (out_bf16)
        reinterpret_cast<uint16_t *>(y)[i] = (uint16_t)f32_to_bf16_rne(v);
    else
        y[i] = v;
}

}  // namespace convfwd
