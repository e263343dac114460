// conv3x3_common.h -- device helpers shared by the 3x3 stride-1 kernels and
// the streaming pointwise kernel (LDS copies, waits, operand packing).
#pragma once

#include "mfma_common.h"

namespace convfwd {

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// 16-byte halves of a 32-byte weight row (one output channel, 16 input
// channels) are swapped on bit 2 xor bit 3 of the row, so 16-byte accesses of
// 8 (32 banks) or 16 (64 banks) consecutive rows reach distinct banks.
__device__ __forceinline__ int wswz(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

// lo 16 bits from half `ha` of a, hi 16 bits from half `hb` of b (one v_perm_b32).
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, int ha, uint32_t b, int hb) {
    const uint32_t sel = (uint32_t)(2 * ha) | ((uint32_t)(2 * ha + 1) << 8) |
                         ((uint32_t)(4 + 2 * hb) << 16) | ((uint32_t)(5 + 2 * hb) << 24);
    return __builtin_amdgcn_perm(b, a, sel);
}

// s_waitcnt with only the vector-memory counter limited to n (n < 64).
#define CONV3X3_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))


// One wave copies 1 KB (64 lanes x 16 bytes) from buffer `rsrc` at byte
// offset soff + 16*lane straight into LDS at `dst` + 16*lane.  Issued as
// inline assembly: the instruction has no register result, and the
// compiler's own waits after the builtin form would also wait for unrelated
// loads in flight.  The caller waits (vmcnt) before the barrier that
// publishes the data; nothing reads the target before that barrier.
__device__ __forceinline__ void dma_1k(lds_u8 *dst, __amdgpu_buffer_rsrc_t rsrc, uint32_t lane16, int soff) {
    const uint32_t m0v = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(m0v)), "v"(lane16), "s"(rsrc),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "m0", "memory");
}

}  // namespace convfwd
