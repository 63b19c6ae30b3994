// Device helpers shared by the gfx950 kernels: bf16 packing, wave64 and
// workgroup reductions, and the launch constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bloom {

constexpr int kWave = 64;
constexpr int kMaxBlock = 1024;
constexpr int kMaxWaves = kMaxBlock / kWave;

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the upper half of an fp32, so widening is a shift;
// narrowing uses gfx950's v_cvt_pk_bf16_f32 (round to nearest even, NaN
// quieted), reached through clang's __bf16 vector conversion.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint4 pack8(const float f[8]) {
  uint4 r;
  r.x = pack2(f[0], f[1]);
  r.y = pack2(f[2], f[3]);
  r.z = pack2(f[4], f[5]);
  r.w = pack2(f[6], f[7]);
  return r;
}

// ---------------------------------------------------------------------------
// Streaming (non-temporal) 8- and 16-byte loads and stores.  Data that is read
// or written once per pass and not touched again until gigabytes of other
// traffic have gone by gains nothing from L2 or the Infinity Cache; marking
// both its loads and its stores non-temporal raises the flat streams of the
// optimizer from ~6.0 to ~6.6 TB/s on MI355X (marking only one side does not).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4 ld_nt(const float4* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st_nt(float4* p, const float4& x) {
  const f32x4_t v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void st_nt(uint4* p, const uint4& x) {
  const u32x4_t v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st_nt(uint2* p, const uint2& x) {
  const u32x2_t v = {x.x, x.y};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}

// ---------------------------------------------------------------------------
// Wave64 all-reductions.  Inside each 16-lane DPP row: quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror, row_mirror -- after these every lane
// holds its row's total (each step pairs every lane with a distinct partner,
// and a+b == b+a, so all lanes of a row agree bit for bit).  The four row
// totals are then read as scalars and combined in a fixed order, so every
// lane gets the same, order-determined result.  Call from wave-uniform
// control flow with all 64 lanes active.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_lanes(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return (row_lanes(v, 0) + row_lanes(v, 16)) + (row_lanes(v, 32) + row_lanes(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return fmaxf(fmaxf(row_lanes(v, 0), row_lanes(v, 16)), fmaxf(row_lanes(v, 32), row_lanes(v, 48)));
}

// Two sums at once (one pass of DPP for each; shares the readlane step).
__device__ __forceinline__ void wave_sum2(float& a, float& b) {
  a = wave_sum(a);
  b = wave_sum(b);
}

// FP64 wave sum through cross-lane shuffles (used once per workgroup).
__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Workgroup all-reductions over `nwaves` waves (all threads of the group
// participate).  `lds` needs kMaxWaves floats (2x for the pair version).
// Wave totals are combined in wave order, identically in every thread.
__device__ __forceinline__ float block_sum(float v, float* lds, int nwaves) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int k = 0; k < nwaves; ++k) s += lds[k];
  __syncthreads();
  return s;
}

__device__ __forceinline__ float block_max(float v, float* lds, int nwaves) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
  __syncthreads();
  float s = -INFINITY;
  for (int k = 0; k < nwaves; ++k) s = fmaxf(s, lds[k]);
  __syncthreads();
  return s;
}

__device__ __forceinline__ void block_sum2(float& a, float& b, float* lds, int nwaves) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lds[w] = a;
    lds[kMaxWaves + w] = b;
  }
  __syncthreads();
  float sa = 0.f, sb = 0.f;
  for (int k = 0; k < nwaves; ++k) {
    sa += lds[k];
    sb += lds[kMaxWaves + k];
  }
  __syncthreads();
  a = sa;
  b = sb;
}

}  // namespace bloom
