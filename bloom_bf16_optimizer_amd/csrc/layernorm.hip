// LayerNorm forward and backward for gfx950.
//
// What is computed: the fused LayerNorm of page "BLOOM 176B 训练技术概览",
// section "融合 CUDA 核", also used as the embedding LayerNorm of "架构微调".
// Per row of width H: mu = sum(x)/H, var = sum((x-mu)^2)/H,
// r = 1/sqrt(var+eps), y = (x-mu)*r*gamma + beta; backward
// dx = r*(g - mean(g) - x_hat*mean(g*x_hat)) with g = dy*gamma,
// dgamma = sum_rows(dy*x_hat), dbeta = sum_rows(dy).
//
// Layout and mapping.  Rows are contiguous bf16; a "row team" of `tpr`
// threads owns a row and each thread holds up to NV 16-byte vectors (8 bf16)
// of it in registers, vector v = t + k*tpr (k < NV), so one row is read from
// HBM exactly once with fully coalesced 16-byte loads.  tpr == 64 means one
// wave per row (reductions in DPP, several rows per workgroup); otherwise the
// whole workgroup is the team and reductions go wave -> LDS.
//
// The backward keeps per-thread FP32 column sums of dy*x_hat and dy for the
// columns it owns while its team walks a strided set of rows, combines the
// teams of a workgroup in LDS, and writes one FP32 partial row per workgroup;
// colsum_kernel (colsum.hip) adds the partial rows in a fixed order.
#include <mutex>

#include "device_common.h"
#include "host_common.h"
#include "launch_plan.h"

// Scratch of bloom_layernorm_bwd_noalloc: its column partial rows live here
// instead of in a caller workspace.  One copy per device, held until the
// process ends; every call on a device shares it.
static __device__ __align__(256) unsigned char scratch[BLOOM_NOALLOC_SCRATCH_BYTES];

namespace bloom {
namespace {

constexpr int kGammaLdsMax = 16384;  // widest row whose gamma the backward stages in LDS (32 KiB)

// Packed bf16 sum of two vectors: FP32 add, one rounding to nearest even (for
// bf16 operands the FP32 sum is exact unless the exponents are 16+ apart, and
// then it lies within 2^-16 of the larger operand, far from a bf16 tie, so the
// result is the exact sum correctly rounded).
__device__ __forceinline__ uint4 add_bf16x8(const uint4& a, const uint4& b) {
  float fa[8], fb[8];
  unpack8(a, fa);
  unpack8(b, fb);
#pragma unroll
  for (int e = 0; e < 8; ++e) fa[e] += fb[e];
  return pack8(fa);
}

// RES: the residual form -- h = bf16(x + res) is formed on load, written to
// h_out, and normalised in place of x.  WAVE: one wave per row (tpr == 64);
// otherwise the workgroup is the row team.  EXACT: the team covers the row
// with no idle lane (tpr * NV == vecs), so no vector needs a bounds guard,
// and a block team is exactly MAXB threads, so its width is a constant.
// Both are template parameters, not run-time branches: each kernel holds only
// its own reduction and index arithmetic.  WPE: the waves per SIMD the
// register allocation must allow (1: no constraint).  At H = 14336 (256 x 7)
// the block-team kernel fits 95 VGPRs with WPE = 5, five one-row workgroups
// per compute unit instead of four.  That wins while the whole launch is
// short and loses on long ones (same process, outputs bit-identical, against
// the four-wave kernel without the exact cover): [2048, 14336] 22.5 against
// 23.8 us, [2560] 30.8 against 29.5, [3072] 34.0 against 34.0, [4096] 44.0
// against 43.5, [8192] 83.9 against 82.6.  So the five-wave kernel runs when
// the rows fit in two rounds of four one-row workgroups per compute unit.
template <int NV, int MAXB, bool RES, bool WAVE, bool EXACT, int WPE>
__global__ __launch_bounds__(MAXB) __attribute__((amdgpu_waves_per_eu(WPE)))
void ln_fwd_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ res, uint4* __restrict__ h_out,
    const uint4* __restrict__ gamma, const uint4* __restrict__ beta,
    uint4* __restrict__ y, float* __restrict__ mean, float* __restrict__ rstd, int64_t rows,
    int vecs_arg, int tpr_arg, float hidden, float eps) {
  __shared__ float lds[kMaxWaves];
  constexpr bool wave_rows = WAVE;
  const int tpr = WAVE ? kWave : (EXACT ? MAXB : tpr_arg);
  const int vecs = EXACT ? tpr * NV : vecs_arg;
  const int t = wave_rows ? (int)(threadIdx.x & (kWave - 1)) : (int)threadIdx.x;
  const int64_t row = wave_rows
                          ? (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave
                          : (int64_t)blockIdx.x;
  if (row >= rows) return;  // uniform over the team
  const int nwaves = blockDim.x / kWave;
  const uint4* xr = x + row * vecs;

  // gamma and beta are read after the statistics: they are shared by every row
  // (served from L2), and keeping them out of registers during the reductions
  // lets more rows be in flight per compute unit.
  uint4 xv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    xv[k] = (EXACT || v < vecs) ? ld_nt(xr + v) : make_uint4(0u, 0u, 0u, 0u);
  }
  if (RES) {
    uint4 rv[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = t + k * tpr;
      rv[k] = (EXACT || v < vecs) ? ld_nt(res + row * vecs + v) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = t + k * tpr;
      xv[k] = add_bf16x8(xv[k], rv[k]);
      if (EXACT || v < vecs) st_nt(h_out + row * vecs + v, xv[k]);
    }
  }

  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float f[8];
    unpack8(xv[k], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += f[e];
  }
  s = wave_rows ? wave_sum(s) : block_sum(s, lds, nwaves);
  const float mu = s / hidden;

  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (EXACT || t + k * tpr < vecs) {
      float f[8];
      unpack8(xv[k], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = f[e] - mu;
        q = fmaf(d, d, q);
      }
    }
  }
  q = wave_rows ? wave_sum(q) : block_sum(q, lds, nwaves);
  const float r = 1.0f / sqrtf(q / hidden + eps);

  uint4* yr = y + row * vecs;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    if (EXACT || v < vecs) {
      float f[8], g[8], b[8], o[8];
      unpack8(xv[k], f);
      unpack8(gamma[v], g);
      unpack8(beta[v], b);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf((f[e] - mu) * r, g[e], b[e]);
      st_nt(yr + v, pack8(o));
    }
  }
  if (t == 0) {
    mean[row] = mu;
    rstd[row] = r;
  }
}

// partial: [gridDim.x][2*H] fp32 -- dgamma partials then dbeta partials.
// Dynamic LDS: gamma as bf16 (2*H bytes, when H <= kGammaLdsMax), then, in
// wave mode with several teams, 2*H floats for combining the teams' column sums.
// RES: the residual form -- dres (the gradient reaching x through the
// residual stream) is added to dx in FP32 before the rounding.
template <int NV, int MAXB, bool RES>
__global__ __launch_bounds__(MAXB) void ln_bwd_kernel(
    const uint4* __restrict__ dy, const uint4* __restrict__ x, const uint4* __restrict__ dres,
    const uint4* __restrict__ gamma, const float* __restrict__ mean,
    const float* __restrict__ rstd, uint4* __restrict__ dx, float* __restrict__ partial,
    int64_t rows, int vecs, int tpr, float hidden) {
  __shared__ float lds[2 * kMaxWaves];
  extern __shared__ uint4 dyn_lds[];
  const bool gamma_staged = vecs * 8 <= kGammaLdsMax;
  uint4* gamma_lds = dyn_lds;                                                  // [vecs]
  float* combine = reinterpret_cast<float*>(dyn_lds + (gamma_staged ? vecs : 0));  // [2*H] (wave mode)
  const bool wave_rows = (tpr == kWave);
  const int teams = wave_rows ? (int)(blockDim.x / kWave) : 1;
  const int team = wave_rows ? (int)(threadIdx.x / kWave) : 0;
  const int t = wave_rows ? (int)(threadIdx.x & (kWave - 1)) : (int)threadIdx.x;
  const int nwaves = blockDim.x / kWave;
  const int64_t team_count = (int64_t)gridDim.x * teams;

  // gamma is shared by every row: staged once in LDS, so reading it in the
  // row loop does not wait on the vector-memory counter that also tracks the
  // next row's prefetched loads.  (Rows wider than kGammaLdsMax read it from
  // global memory instead.)
  const uint4* gsrc = gamma;
  if (gamma_staged) {
    for (int v = threadIdx.x; v < vecs; v += blockDim.x) gamma_lds[v] = gamma[v];
    __syncthreads();
  }

  float dg[NV][8], db[NV][8];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dg[k][e] = 0.f;
      db[k][e] = 0.f;
    }
  }

  // Software pipelining: the next row's dy and x are requested before the
  // current row's reductions, so each team keeps two rows of loads in flight.
  int64_t row = (int64_t)blockIdx.x * teams + team;
  uint4 dv[NV], xv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    if (row < rows && v < vecs) {
      dv[k] = ld_nt(dy + row * vecs + v);
      xv[k] = ld_nt(x + row * vecs + v);
    } else {
      dv[k] = make_uint4(0u, 0u, 0u, 0u);
      xv[k] = dv[k];
    }
  }
  for (; row < rows; row += team_count) {
    const int64_t next = row + team_count;
    uint4 dn[NV], xn[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = t + k * tpr;
      if (next < rows && v < vecs) {
        dn[k] = ld_nt(dy + next * vecs + v);
        xn[k] = ld_nt(x + next * vecs + v);
      } else {
        dn[k] = make_uint4(0u, 0u, 0u, 0u);
        xn[k] = dn[k];
      }
    }
    const float mu = mean[row];
    const float r = rstd[row];
    uint4 rv[NV];
    if (RES) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int v = t + k * tpr;
        rv[k] = (v < vecs) ? ld_nt(dres + row * vecs + v) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // First pass: the row sums of g and g*x_hat, and this row's share of the
    // column sums dgamma += dy*x_hat, dbeta += dy (they need no row statistic).
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = t + k * tpr;
      if (v < vecs) {
        float d[8], f[8], g[8];
        unpack8(dv[k], d);
        unpack8(xv[k], f);
        unpack8(gamma_staged ? gamma_lds[v] : gsrc[v], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gg = d[e] * g[e];
          const float xh = (f[e] - mu) * r;
          sg += gg;
          sgx = fmaf(gg, xh, sgx);
          dg[k][e] = fmaf(d[e], xh, dg[k][e]);
          db[k][e] += d[e];
        }
      }
    }
    if (wave_rows) {
      wave_sum2(sg, sgx);
    } else {
      block_sum2(sg, sgx, lds, nwaves);
    }
    const float mg = sg / hidden;
    const float mgx = sgx / hidden;
    // Second pass: dx from the same registers.
    uint4* dxr = dx + row * vecs;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = t + k * tpr;
      if (v < vecs) {
        float d[8], f[8], g[8], o[8];
        unpack8(dv[k], d);
        unpack8(xv[k], f);
        unpack8(gamma_staged ? gamma_lds[v] : gsrc[v], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (f[e] - mu) * r;
          o[e] = r * (d[e] * g[e] - mg - xh * mgx);
        }
        if (RES) {
          float q[8];
          unpack8(rv[k], q);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += q[e];
        }
        st_nt(dxr + v, pack8(o));
      }
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      dv[k] = dn[k];
      xv[k] = xn[k];
    }
  }

  const int hidden_i = vecs * 8;
  float* out = partial + (int64_t)blockIdx.x * 2 * hidden_i;
  if (teams == 1) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = t + k * tpr;
      if (v < vecs) {
        float4* og = reinterpret_cast<float4*>(out + v * 8);
        float4* ob = reinterpret_cast<float4*>(out + hidden_i + v * 8);
        og[0] = make_float4(dg[k][0], dg[k][1], dg[k][2], dg[k][3]);
        og[1] = make_float4(dg[k][4], dg[k][5], dg[k][6], dg[k][7]);
        ob[0] = make_float4(db[k][0], db[k][1], db[k][2], db[k][3]);
        ob[1] = make_float4(db[k][4], db[k][5], db[k][6], db[k][7]);
      }
    }
    return;
  }
  // Several wave-teams: add them in team order in LDS, then write one row.
  for (int turn = 0; turn < teams; ++turn) {
    if (team == turn) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int v = t + k * tpr;
        if (v < vecs) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int c = v * 8 + e;
            combine[c] = (turn == 0) ? dg[k][e] : combine[c] + dg[k][e];
            combine[hidden_i + c] = (turn == 0) ? db[k][e] : combine[hidden_i + c] + db[k][e];
          }
        }
      }
    }
    __syncthreads();
  }
  for (int c = threadIdx.x * 4; c < 2 * hidden_i; c += blockDim.x * 4)
    *reinterpret_cast<float4*>(out + c) = *reinterpret_cast<const float4*>(combine + c);
}

// ---------------------------------------------------------------------------
// Streaming backward for rows that one workgroup covers exactly (tpr*NV ==
// vecs, NV <= 2): the path of the BLOOM-176B hidden sizes.
//
// Each wave streams its own lanes' share of the next two rows straight into
// LDS with global_load_lds_dwordx4 (16 bytes per lane, written at
// m0 + lane*16), so two rows are in flight while a third is computed from
// registers.  A lane only ever reads back the 16-byte slots its own transfer
// wrote, so the ring needs no barrier: a per-wave s_waitcnt on the
// vector-memory counter is enough.  The transfers and the waits are inline
// assembly with exact counts, because the compiler's own wait insertion
// drains the whole counter at loop back-edges, which would serialise the rows
// again.  Every vector-memory instruction a wave issues in the row loop is
// accounted for: per row 2*NV row transfers, NV dx stores and, in the
// residual form, NV transfers of the row's dres (the row statistics are
// scalar loads, counted by lgkmcnt instead).
//
// LDS (dynamic, uint4 units, W = waves of the team):
//   ring [slot 2][tensor 2 (dy, x)][k NV][wave W][lane 64], then, with RES,
//   dres [k NV][wave W][lane 64] (one row deep: requested at the start of a
//   row, read after its reductions).
// The arithmetic, its order and the partial-row layout are exactly those of
// ln_bwd_kernel for the same team, so both produce identical bits.
typedef uint32_t u32x4_lds_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint4 lds_uint4;

__device__ __forceinline__ uint32_t lds_offset(const lds_uint4* p) { return (uint32_t)(uintptr_t)p; }

// One 16-byte-per-lane transfer from global memory into LDS at m0 + lane*16.
__device__ __forceinline__ void dma16(const uint4* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Requests `src_row` (a row of `vecs` vectors; or, when !live, a harmless
// re-read of gamma) for this wave's lanes into LDS at `base`, laid out
// [k NV][wave W][lane 64].
template <int NV>
__device__ __forceinline__ void lds_issue(lds_uint4* base, const uint4* __restrict__ src_row,
                                          const uint4* __restrict__ gamma, bool live, int t, int tpr,
                                          int w, int nwaves) {
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    const uint4* src = live ? src_row + v : gamma + v;
    dma16(src, __builtin_amdgcn_readfirstlane(lds_offset(base + (k * nwaves + w) * kWave)));
  }
}

// Reads this lane's NV slots.  The reads and their lgkmcnt wait are ONE asm
// statement: an asm output counts as defined when its statement ends, so a
// wait in a separate statement would let the compiler schedule uses of the
// registers before the data has arrived.  Early-clobber outputs keep a
// destination from sharing a register with an address still to be read.
template <int NV>
__device__ __forceinline__ void lds_read(const lds_uint4* base, int w, int lane, int nwaves, uint4 (&out)[NV]) {
  static_assert(NV == 1 || NV == 2, "lds_read handles one or two slots");
  u32x4_lds_t r0, r1;
  const uint32_t a0 = lds_offset(base + (0 * nwaves + w) * kWave + lane);
  if (NV == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r0) : "v"(a0) : "memory");
  } else {
    const uint32_t a1 = lds_offset(base + (1 * nwaves + w) * kWave + lane);
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r0), "=&v"(r1)
                 : "v"(a0), "v"(a1)
                 : "memory");
  }
  out[0] = make_uint4(r0.x, r0.y, r0.z, r0.w);
  if (NV == 2) out[NV - 1] = make_uint4(r1.x, r1.y, r1.z, r1.w);
}

template <int NV, bool RES>
__global__ __launch_bounds__(kMaxBlock) void ln_bwd_stream_kernel(
    const uint4* __restrict__ dy, const uint4* __restrict__ x, const uint4* __restrict__ dres,
    const uint4* __restrict__ gamma, const float* __restrict__ mean,
    const float* __restrict__ rstd, uint4* __restrict__ dx, float* __restrict__ partial,
    int64_t rows, int vecs, float hidden) {
  extern __shared__ uint4 stream_lds[];
  __shared__ float red[2][2 * kMaxWaves];
  const int t = threadIdx.x, tpr = blockDim.x, nwaves = tpr / kWave;
  const int w = t / kWave, lane = t & (kWave - 1);
  lds_uint4* ring = (lds_uint4*)stream_lds;
  const int tensor_stride = NV * nwaves * kWave;  // uint4 per [k][wave][lane] block
  lds_uint4* dres_slot = ring + 4 * tensor_stride;
  const int64_t first = blockIdx.x, stride = gridDim.x;
  const int count = (int)((rows - first + stride - 1) / stride);  // >= 1: grid <= rows

  // gamma lives in registers; the empty asm makes its loads complete here,
  // before any transfer is issued, so no later wait has to cover them.
  uint4 g[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) g[k] = gamma[t + k * tpr];
#pragma unroll
  for (int k = 0; k < NV; ++k) asm volatile("" : "+v"(g[k].x), "+v"(g[k].y), "+v"(g[k].z), "+v"(g[k].w));
  float dg[NV][8], db[NV][8];
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) dg[k][e] = db[k][e] = 0.f;

  // slot s, tensor q at ring + (2*s + q) * tensor_stride
#pragma unroll
  for (int s0 = 0; s0 < 2; ++s0) {
    const int64_t row = first + s0 * stride;
    const bool live = s0 < count;
    lds_issue<NV>(ring + (2 * s0 + 0) * tensor_stride, dy + row * vecs, gamma, live, t, tpr, w, nwaves);
    lds_issue<NV>(ring + (2 * s0 + 1) * tensor_stride, x + row * vecs, gamma, live, t, tpr, w, nwaves);
  }
  for (int i = 0; i < count; ++i) {
    const int slot = i & 1;
    // Row i's transfers are done once no more than the operations issued after
    // them are outstanding.  Per row: R = dres transfers (NV, residual form
    // only), T = 2*NV row transfers, S = NV stores.  Row 0: T (row 1's);
    // row 1: R + T + S of row 0; later: S(i-2) + R + T + S of row i-1.
    if (i >= 2)
      wait_vmem<(RES ? 5 : 4) * NV>();
    else if (i == 1)
      wait_vmem<(RES ? 4 : 3) * NV>();
    else
      wait_vmem<2 * NV>();
    uint4 dv[NV], xv[NV];
    lds_read<NV>(ring + (2 * slot + 0) * tensor_stride, w, lane, nwaves, dv);
    lds_read<NV>(ring + (2 * slot + 1) * tensor_stride, w, lane, nwaves, xv);
    const int64_t row = first + (int64_t)i * stride;
    if (RES) lds_issue<NV>(dres_slot, dres + row * vecs, gamma, true, t, tpr, w, nwaves);
    // The slot is free again: request row i+2 into it (a dummy past the end,
    // so that every iteration issues the same number of operations).
    {
      const int64_t nrow = first + (int64_t)(i + 2) * stride;
      const bool live = i + 2 < count;
      lds_issue<NV>(ring + (2 * slot + 0) * tensor_stride, dy + nrow * vecs, gamma, live, t, tpr, w, nwaves);
      lds_issue<NV>(ring + (2 * slot + 1) * tensor_stride, x + nrow * vecs, gamma, live, t, tpr, w, nwaves);
    }
    const float mu = mean[row];
    const float r = rstd[row];
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float d[8], f[8], gg[8];
      unpack8(dv[k], d);
      unpack8(xv[k], f);
      unpack8(g[k], gg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = d[e] * gg[e];
        const float xh = (f[e] - mu) * r;
        sg += p;
        sgx = fmaf(p, xh, sgx);
        dg[k][e] = fmaf(d[e], xh, dg[k][e]);
        db[k][e] += d[e];
      }
    }
    // Workgroup sums with one barrier: the two halves of `red` alternate, and
    // a wave can only write a half again after every wave has passed the next
    // barrier, i.e. after all of them have read it.
    sg = wave_sum(sg);
    sgx = wave_sum(sgx);
    float* rr = red[slot];
    if (lane == 0) {
      rr[w] = sg;
      rr[kMaxWaves + w] = sgx;
    }
    __syncthreads();
    float a = 0.f, b = 0.f;
    for (int k = 0; k < nwaves; ++k) {
      a += rr[k];
      b += rr[kMaxWaves + k];
    }
    const float mg = a / hidden;
    const float mgx = b / hidden;
    uint4 qv[NV];
    if (RES) {
      wait_vmem<2 * NV>();  // this row's dres: only row i+2's transfers were issued after it
      lds_read<NV>(dres_slot, w, lane, nwaves, qv);
    }
    uint4* dxr = dx + row * vecs;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float d[8], f[8], gg[8], o[8];
      unpack8(dv[k], d);
      unpack8(xv[k], f);
      unpack8(g[k], gg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xh = (f[e] - mu) * r;
        o[e] = r * (d[e] * gg[e] - mg - xh * mgx);
      }
      if (RES) {
        float q[8];
        unpack8(qv[k], q);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += q[e];
      }
      st_nt(dxr + t + k * tpr, pack8(o));
    }
    asm volatile("" ::: "memory");  // keeps the stores inside this iteration's count
  }
  // The trailing dummy transfers must land before the workgroup's LDS is released.
  wait_vmem<0>();

  const int hidden_i = vecs * 8;
  float* out = partial + (int64_t)blockIdx.x * 2 * hidden_i;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    float4* og = reinterpret_cast<float4*>(out + v * 8);
    float4* ob = reinterpret_cast<float4*>(out + hidden_i + v * 8);
    og[0] = make_float4(dg[k][0], dg[k][1], dg[k][2], dg[k][3]);
    og[1] = make_float4(dg[k][4], dg[k][5], dg[k][6], dg[k][7]);
    ob[0] = make_float4(db[k][0], db[k][1], db[k][2], db[k][3]);
    ob[1] = make_float4(db[k][4], db[k][5], db[k][6], db[k][7]);
  }
}

constexpr size_t kStreamLdsMax = 160 * 1024 - 2 * 2 * kMaxWaves * sizeof(float);

inline size_t stream_lds_bytes(const RowPlan& p, bool res) {
  return (size_t)(4 + (res ? 1 : 0)) * p.nv * (p.tpr / kWave) * kWave * sizeof(uint4);
}

// The streaming backward applies when a block-mode team covers the row with
// no idle lane, at most two vectors per thread, and its ring fits in LDS.
inline bool use_stream_bwd(const RowPlan& p, int vecs, bool res) {
  return p.tpr > kWave && p.block == p.tpr && p.tpr <= kMaxBlock && p.nv <= 2 && p.tpr * p.nv == vecs &&
         stream_lds_bytes(p, res) <= kStreamLdsMax;
}

template <int NV, int MAXB, bool RES>
void launch_fwd(const RowPlan& p, hipStream_t s, const uint4* x, const uint4* res, uint4* h,
                const uint4* g, const uint4* b, uint4* y, float* mean, float* rstd, int64_t rows,
                int vecs, float eps) {
  const bool exact = p.tpr * NV == vecs && (p.tpr == kWave || p.tpr == MAXB);
  const bool short_launch = rows <= (int64_t)8 * device_cu_count();
#define BLOOM_LN_FWD(WAVE, EXACT, WPE)                                                                          \
  hipLaunchKernelGGL((ln_fwd_kernel<NV, MAXB, RES, WAVE, EXACT, WPE>), dim3(p.grid), dim3(p.block), 0, s, x, res, h, \
                     g, b, y, mean, rstd, rows, vecs, p.tpr, (float)(vecs * 8), eps)
  if (p.tpr == kWave) {
    if (exact) BLOOM_LN_FWD(true, true, 1); else BLOOM_LN_FWD(true, false, 1);
  } else if (exact && NV == 7 && MAXB == 256 && short_launch) {
    BLOOM_LN_FWD(false, true, 5);
  } else if (NV == 7 && MAXB == 256) {
    BLOOM_LN_FWD(false, false, 1);
  } else {
    if (exact) BLOOM_LN_FWD(false, true, 1); else BLOOM_LN_FWD(false, false, 1);
  }
#undef BLOOM_LN_FWD
}

template <int NV, int MAXB, bool RES>
void launch_bwd(const RowPlan& p, hipStream_t s, const uint4* dy, const uint4* x, const uint4* dres,
                const uint4* g, const float* mean, const float* rstd, uint4* dx, float* partial,
                int64_t rows, int vecs, size_t lds_bytes) {
  hipLaunchKernelGGL((ln_bwd_kernel<NV, MAXB, RES>), dim3(p.grid), dim3(p.block), lds_bytes, s, dy, x, dres, g,
                     mean, rstd, dx, partial, rows, vecs, p.tpr, (float)(vecs * 8));
}

bloom_status check_rows(int64_t rows, int64_t hidden) {
  BLOOM_REQUIRE(rows >= 0, BLOOM_ERR_SHAPE, "rows = %lld is negative", (long long)rows);
  BLOOM_REQUIRE(hidden >= 8 && hidden <= BLOOM_MAX_HIDDEN && hidden % 8 == 0, BLOOM_ERR_SHAPE,
                "hidden = %lld must be a multiple of 8 in [8, %d]", (long long)hidden,
                BLOOM_MAX_HIDDEN);
  BLOOM_REQUIRE(rows <= (int64_t(1) << 40) / hidden, BLOOM_ERR_SHAPE, "rows*hidden too large");
  return BLOOM_OK;
}

// Shared by the plain and the residual forward (res == NULL: plain).
template <bool RES>
bloom_status layernorm_fwd_impl(const char* name, const bloom_bf16* x, const bloom_bf16* res,
                                bloom_bf16* h, const bloom_bf16* gamma, const bloom_bf16* beta,
                                bloom_bf16* y, float* mean, float* rstd, int64_t rows, int64_t hidden,
                                float eps, hipStream_t stream) {
  if (bloom_status st = check_rows(rows, hidden)) return st;
  BLOOM_REQUIRE(eps > 0.f && eps < INFINITY, BLOOM_ERR_HPARAM, "eps must be positive and finite");
  if (rows == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(x);
  if (RES) {
    BLOOM_REQUIRE_PTR(res);
    BLOOM_REQUIRE_PTR(h);
  }
  BLOOM_REQUIRE_PTR(gamma);
  BLOOM_REQUIRE_PTR(beta);
  BLOOM_REQUIRE_PTR(y);
  BLOOM_REQUIRE_PTR(mean);
  BLOOM_REQUIRE_PTR(rstd);
  const int vecs = (int)(hidden / 8);
  const RowPlan p = plan_rows_fwd(rows, vecs);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const uint4* rv = reinterpret_cast<const uint4*>(res);
  uint4* hv = reinterpret_cast<uint4*>(h);
  const uint4* gv = reinterpret_cast<const uint4*>(gamma);
  const uint4* bv = reinterpret_cast<const uint4*>(beta);
  uint4* yv = reinterpret_cast<uint4*>(y);
#define CALL(NV, MAXB) launch_fwd<NV, MAXB, RES>(p, stream, xv, rv, hv, gv, bv, yv, mean, rstd, rows, vecs, eps)
  BLOOM_ROW_DISPATCH(p, CALL);
#undef CALL
  return launch_status(name);
}

// Shared by the plain and the residual backward (dres == NULL: plain).
template <bool RES>
bloom_status layernorm_bwd_impl(const char* name, const bloom_bf16* dy, const bloom_bf16* x,
                                const bloom_bf16* dres, const bloom_bf16* gamma, const float* mean,
                                const float* rstd, bloom_bf16* dx, bloom_bf16* dgamma, bloom_bf16* dbeta,
                                void* workspace, size_t workspace_bytes, int64_t rows, int64_t hidden,
                                hipStream_t stream) {
  if (bloom_status st = check_rows(rows, hidden)) return st;
  if (rows == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(dy);
  BLOOM_REQUIRE_PTR(x);
  if (RES) BLOOM_REQUIRE_PTR(dres);
  BLOOM_REQUIRE_PTR(gamma);
  BLOOM_REQUIRE_PTR(mean);
  BLOOM_REQUIRE_PTR(rstd);
  BLOOM_REQUIRE_PTR(dx);
  BLOOM_REQUIRE_PTR(dgamma);
  BLOOM_REQUIRE_PTR(dbeta);
  BLOOM_REQUIRE(workspace != nullptr, BLOOM_ERR_WORKSPACE, "workspace is NULL");
  BLOOM_REQUIRE(aligned16(workspace), BLOOM_ERR_ALIGN, "workspace is not 16-byte aligned");
  const int vecs = (int)(hidden / 8);
  const RowPlan p = plan_rows_bwd(rows, vecs, device_cu_count());
  const size_t need = (size_t)p.grid * 2 * (size_t)hidden * sizeof(float);
  BLOOM_REQUIRE(workspace_bytes >= need, BLOOM_ERR_WORKSPACE,
                "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  float* partial = static_cast<float*>(workspace);
  const uint4* dyv = reinterpret_cast<const uint4*>(dy);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const uint4* rv = reinterpret_cast<const uint4*>(dres);
  const uint4* gv = reinterpret_cast<const uint4*>(gamma);
  uint4* dxv = reinterpret_cast<uint4*>(dx);
  if (use_stream_bwd(p, vecs, RES)) {
    const size_t lds = stream_lds_bytes(p, RES);
    if (p.nv == 1)
      hipLaunchKernelGGL((ln_bwd_stream_kernel<1, RES>), dim3(p.grid), dim3(p.block), lds, stream, dyv, xv, rv,
                         gv, mean, rstd, dxv, partial, rows, vecs, (float)hidden);
    else
      hipLaunchKernelGGL((ln_bwd_stream_kernel<2, RES>), dim3(p.grid), dim3(p.block), lds, stream, dyv, xv, rv,
                         gv, mean, rstd, dxv, partial, rows, vecs, (float)hidden);
  } else {
    const size_t lds = (hidden <= kGammaLdsMax ? 2 * (size_t)hidden : 0) +
                       ((p.tpr == kWave && p.block > kWave) ? 2 * (size_t)hidden * sizeof(float) : 0);
#define CALL(NV, MAXB) \
  launch_bwd<NV, MAXB, RES>(p, stream, dyv, xv, rv, gv, mean, rstd, dxv, partial, rows, vecs, lds)
    BLOOM_ROW_DISPATCH(p, CALL);
#undef CALL
  }
  if (bloom_status st = launch_status(name)) return st;
  launch_colsum(partial, p.grid, 2 * hidden, hidden, dgamma, dbeta, stream);
  return launch_status(name);
}

}  // namespace
}  // namespace bloom

using namespace bloom;

extern "C" bloom_status bloom_layernorm_fwd(const bloom_bf16* x, const bloom_bf16* gamma,
                                            const bloom_bf16* beta, bloom_bf16* y, float* mean,
                                            float* rstd, int64_t rows, int64_t hidden, float eps,
                                            hipStream_t stream) {
  clear_error();
  return layernorm_fwd_impl<false>("bloom_layernorm_fwd", x, nullptr, nullptr, gamma, beta, y, mean, rstd,
                                   rows, hidden, eps, stream);
}

extern "C" bloom_status bloom_layernorm_residual_fwd(const bloom_bf16* x, const bloom_bf16* residual,
                                                     const bloom_bf16* gamma, const bloom_bf16* beta,
                                                     bloom_bf16* h, bloom_bf16* y, float* mean,
                                                     float* rstd, int64_t rows, int64_t hidden, float eps,
                                                     hipStream_t stream) {
  clear_error();
  return layernorm_fwd_impl<true>("bloom_layernorm_residual_fwd", x, residual, h, gamma, beta, y, mean,
                                  rstd, rows, hidden, eps, stream);
}

extern "C" size_t bloom_layernorm_bwd_workspace_size(int64_t rows, int64_t hidden) {
  if (rows <= 0 || hidden <= 0 || hidden % 8 != 0 || hidden > BLOOM_MAX_HIDDEN) return 0;
  const RowPlan p = plan_rows_bwd(rows, (int)(hidden / 8), device_cu_count());
  return (size_t)p.grid * 2 * (size_t)hidden * sizeof(float);
}

extern "C" bloom_status bloom_layernorm_bwd(const bloom_bf16* dy, const bloom_bf16* x,
                                            const bloom_bf16* gamma, const float* mean,
                                            const float* rstd, bloom_bf16* dx, bloom_bf16* dgamma,
                                            bloom_bf16* dbeta, void* workspace,
                                            size_t workspace_bytes, int64_t rows, int64_t hidden,
                                            hipStream_t stream) {
  clear_error();
  return layernorm_bwd_impl<false>("bloom_layernorm_bwd", dy, x, nullptr, gamma, mean, rstd, dx, dgamma,
                                   dbeta, workspace, workspace_bytes, rows, hidden, stream);
}

namespace bloom {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device of `stream`, looked up once
// per device with that device current.  In host code `scratch` names a host
// stand-in, so only this address may reach a kernel.
bloom_status scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(BLOOM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  hipDevice_t sdev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(BLOOM_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  BLOOM_REQUIRE(sdev == cur, BLOOM_ERR_HPARAM,
                "stream belongs to device %d but device %d is current; make the stream's device current", (int)sdev,
                cur);
  BLOOM_REQUIRE(cur >= 0 && cur < kMaxDevices, BLOOM_ERR_HIP, "device %d beyond the %d supported", cur, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[cur] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(BLOOM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", cur, hipGetErrorString(e));
    g_scratch_ptr[cur] = p;
  }
  *out = g_scratch_ptr[cur];
  return BLOOM_OK;
}

}  // namespace
}  // namespace bloom

extern "C" bloom_status bloom_layernorm_bwd_noalloc(const bloom_bf16* dy, const bloom_bf16* x,
                                                    const bloom_bf16* gamma, const float* mean,
                                                    const float* rstd, bloom_bf16* dx, bloom_bf16* dgamma,
                                                    bloom_bf16* dbeta, int64_t rows, int64_t hidden,
                                                    hipStream_t stream) {
  clear_error();
  if (bloom_status st = check_rows(rows, hidden)) return st;
  if (rows == 0) return BLOOM_OK;
  const size_t need = bloom_layernorm_bwd_workspace_size(rows, hidden);
  BLOOM_REQUIRE(need <= (size_t)BLOOM_NOALLOC_SCRATCH_BYTES, BLOOM_ERR_WORKSPACE,
                "rows = %lld, hidden = %lld need %zu bytes of scratch; the static scratch holds %zu "
                "(use bloom_layernorm_bwd with a workspace)",
                (long long)rows, (long long)hidden, need, (size_t)BLOOM_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (bloom_status st = scratch_address(stream, &ws)) return st;
  return layernorm_bwd_impl<false>("bloom_layernorm_bwd_noalloc", dy, x, nullptr, gamma, mean, rstd, dx, dgamma,
                                   dbeta, ws, (size_t)BLOOM_NOALLOC_SCRATCH_BYTES, rows, hidden, stream);
}

extern "C" bloom_status bloom_layernorm_residual_bwd(const bloom_bf16* dy, const bloom_bf16* dres,
                                                     const bloom_bf16* h, const bloom_bf16* gamma,
                                                     const float* mean, const float* rstd,
                                                     bloom_bf16* dh, bloom_bf16* dgamma,
                                                     bloom_bf16* dbeta, void* workspace,
                                                     size_t workspace_bytes, int64_t rows,
                                                     int64_t hidden, hipStream_t stream) {
  clear_error();
  return layernorm_bwd_impl<true>("bloom_layernorm_residual_bwd", dy, h, dres, gamma, mean, rstd, dh,
                                  dgamma, dbeta, workspace, workspace_bytes, rows, hidden, stream);
}
