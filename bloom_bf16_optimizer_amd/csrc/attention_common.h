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

// ALiBi offset fragments for the score products S^T = K Q^T: k-slots 0..2
// of the lower lane half carry the key's offset in its block (an integer
// < 64, exact in bf16) in kx (kx[1]: the block's second 32 keys), against
// slope/scale split into three bf16 parts in qx; every other slot is zero.
// One more MFMA k-step with them adds offset * slope/scale to every score.
__device__ __forceinline__ void attn_key_offsets(bf16x8_t (&kx)[2], int half, int col) {
  const __bf16 z = (__bf16)0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool on = half == 0 && j < 3;
    kx[0][j] = on ? (__bf16)(float)col : z;
    kx[1][j] = on ? (__bf16)(float)(col + 32) : z;
  }
}
__device__ __forceinline__ bf16x8_t attn_slope_parts(float slope2, float scale2, int half) {
  const float cs = slope2 / scale2;  // slope/scale
  const __bf16 c1 = (__bf16)cs;
  const float r1 = cs - (float)c1;
  const __bf16 c2 = (__bf16)r1;
  const __bf16 c3 = (__bf16)(r1 - (float)c2);
  const __bf16 z = (__bf16)0.0f;
  bf16x8_t qx;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool on = half == 0 && j < 3;
    qx[j] = on ? (j == 0 ? c1 : (j == 1 ? c2 : c3)) : z;
  }
  return qx;
}

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

// Output rows staged through LDS so that they can be stored whole.  A lane
// holds row `row` of a tile of 32-row groups in 32x32 accumulator fragments
// (lane half h: d = 32*dt + 8*g + 4*h + 0..3); attn_stage_row writes them,
// times s, as bf16 into the tile: row r at (r / 32) * GP + (r % 32) * 2D
// bytes (GP: the bytes between 32-row groups), 16-byte chunk c of a row at
// c ^ (r % (D/8)), so that 32 rows written at once and whole rows read
// back are free of bank conflicts.
template <int D>
__device__ __forceinline__ void attn_stage_row(const f32x16_t (&acc)[D / 32], float s, char* tile, int gp, int row,
                                               int half) {
  constexpr int CPR = D / 8;
  // the offsets below are cheap to form here; kept opaque so that the
  // compiler does not hoist them out of the caller's loops into registers
  asm volatile("" : "+v"(row));
  char* rp = tile + (row / 32) * gp + (row % 32) * (2 * D);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t lo = pack2(acc[dt][4 * g] * s, acc[dt][4 * g + 1] * s);
      const uint32_t hi = pack2(acc[dt][4 * g + 2] * s, acc[dt][4 * g + 3] * s);
      const int c = (4 * dt + g) ^ (row % CPR);
      *reinterpret_cast<uint2*>(rp + 16 * c + 8 * half) = make_uint2(lo, hi);
    }
}

// The ROWS staged rows to rows row0 .. of a [*, D] bf16 matrix: NT threads
// store 16 bytes each (whole rows, instead of each lane storing 8-byte
// pieces of 16 rows); rows at or past `valid` are not stored.
template <int D, int ROWS, int NT>
__device__ __forceinline__ void attn_store_staged(const char* tile, int gp, uint2* __restrict__ out, int64_t row0,
                                                  int valid, int t) {
  constexpr int CPR = D / 8;
  constexpr int PER = ROWS * CPR / NT;  // 16-byte chunks per thread
  static_assert(PER >= 1 && ROWS * CPR % NT == 0, "staged rows");
  uint4* o4 = reinterpret_cast<uint4*>(out);
  asm volatile("" : "+v"(t));  // as in attn_stage_row
#pragma unroll
  for (int x = 0; x < PER; ++x) {
    const int chunk = x * NT + t;
    const int row = chunk / CPR, c = chunk % CPR;
    const uint4 val =
        *reinterpret_cast<const uint4*>(tile + (row / 32) * gp + (row % 32) * (2 * D) + 16 * (c ^ (row % CPR)));
    if (row < valid) o4[(row0 + row) * CPR + c] = val;
  }
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
