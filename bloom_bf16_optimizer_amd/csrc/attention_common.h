// Pieces shared by the fused attention kernels (forward and backward) for
// gfx950: the bf16 MFMA tile, LDS vector types, the ALiBi slope table, and
// the direct global-to-LDS transfer.
#pragma once

#include "device_common.h"
#include "host_common.h"

namespace bloom {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct AttnSlopes {
  float s[BLOOM_MAX_HEADS];  // slope_h * log2(e)
};

// v_mfma_f32_32x32x16_bf16: D[32x32] = A[32x16] B[16x32] + C, FP32 accumulate.
// Lane l supplies A row l%32 and B column l%32, each for k = 8*(l/32) .. +7;
// it holds D column l%32, rows 8*(i/4) + 4*(l/32) + i%4 in register i.
__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef __attribute__((address_space(3))) uint4 attn_lds_uint4;
typedef unsigned int attn_u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) attn_u32x4 attn_lds_u32x4;
typedef short attn_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) attn_v4s attn_lds_v4s;

// One 16-byte-per-lane transfer from global memory (wave-uniform base plus
// a 32-bit byte offset per lane) into LDS at m0 + lane*16 (cached: the tiles
// are re-read by other workgroups of the head).  m0 is written only here:
// the compiler uses it for nothing else in these kernels (checked in the
// generated code), so the clobber is only a precaution.
__device__ __forceinline__ void attn_dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}

// Waits for every vector-memory load of the wave, the direct-to-LDS tile
// transfers included (they are inline asm, which the compiler does not
// track), and tells the compiler so.  Without the second, compiler-visible
// wait it takes its own loads issued before a block loop (the next item's
// rows) as still pending and waits for them again at their first use inside
// the loop, on every block; that wait, counted in hardware, also drains the
// next block's transfers issued just before, so the block would wait for its
// successor's tiles.
__device__ __forceinline__ void attn_wait_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited for
}

// A 64-bit pointer made wave-uniform (both halves through readfirstlane), so
// that it can sit in the SGPR pair the transfer instruction takes.
template <typename T>
__device__ __forceinline__ const T* attn_uniform(const T* p) {
  const uint64_t gp = (uint64_t)(uintptr_t)p;
  return (const T*)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(gp >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gp));
}

}  // namespace bloom
