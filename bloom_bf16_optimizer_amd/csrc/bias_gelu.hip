// bias + GeLU forward and backward for gfx950.
//
// What is computed: the bias + GeLU fusion of page "BLOOM 176B 训练技术概览",
// section "融合 CUDA 核" (the GeLU(XA) of the MLP, page "企业官网建设流程全解析",
// section 2.1), in the tanh form of the GELU paper (arXiv:1606.08415):
//   u = x + b,  y = u/2 (1 + tanh(k(u + c u^3))),  k = sqrt(2/pi), c = 0.044715.
// The tanh is rewritten exactly as a logistic function,
//   (1 + tanh(a))/2 = 1/(1 + exp(-2a)),
// so y = u*s with s = 1/(1 + exp2(u*(A + B u^2))), A = -2k*log2(e),
// B = -2kc*log2(e); and the derivative becomes
//   y'(u) = s + 2k*u*s*(1-s)*(1 + 3c u^2).
//
// Mapping: a thread owns one 16-byte column vector (8 columns) for a strip of
// rows, keeping the 8 bias values -- and, in the backward, 8 FP32 dbias sums
// -- in registers.  Consecutive threads own consecutive vectors, so each wave
// reads and writes 1 KiB contiguous per row.  The backward writes one FP32
// partial row per row strip; colsum.hip adds them in strip order.
#include "device_common.h"
#include "host_common.h"
#include "launch_plan.h"

namespace bloom {
namespace {

constexpr double kKd = 0.7978845608028654;
constexpr double kCd = 0.044715;
constexpr double kLog2e = 1.4426950408889634;
constexpr int kUnroll = 4;

struct GeluConsts {
  float a;     // -2k log2(e)
  float b;     // -2kc log2(e)
  float k2;    // 2k
  float c3;    // 3c
};

// s = 1/(1 + exp(-2a)) with the hardware exp2 and reciprocal (each within
// 1 ulp of fp32; exp2 results below 2^-126 flush to 0, which leaves s = 1).
// The element budget is tight: at 8 TB/s the forward has ~20 VALU slots per
// element, so the correctly rounded divide (about 10 instructions) is not used.
__device__ __forceinline__ float logistic_part(float u, const GeluConsts& g) {
  const float t = __builtin_amdgcn_exp2f(u * fmaf(g.b, u * u, g.a));
  return __builtin_amdgcn_rcpf(1.0f + t);
}

__global__ __launch_bounds__(256) void gelu_fwd_kernel(const uint4* __restrict__ x,
                                                       const uint4* __restrict__ bias,
                                                       uint4* __restrict__ y, int64_t rows,
                                                       int vecs, int rows_per_block, GeluConsts g) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= vecs) return;
  float bv[8];
  unpack8(bias[v], bv);
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  for (int64_t r = r0; r < r1; r += kUnroll) {
    uint4 xv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (r + u < r1) xv[u] = ld_nt(x + (r + u) * vecs + v);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (r + u < r1) {
        float f[8], o[8];
        unpack8(xv[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float uu = f[e] + bv[e];
          o[e] = uu * logistic_part(uu, g);
        }
        st_nt(y + (r + u) * vecs + v, pack8(o));
      }
    }
  }
}

// Backward.  A workgroup is 64 column vectors (one per lane) by 4 row groups
// (one per wave): wave w walks rows [r0 + w*RB, r0 + (w+1)*RB) of the block's
// strip, so four times as many waves stream as with one row group per block
// while the strip -- and with it the number of dbias partial rows -- stays at
// 4*RB rows.  The four waves' FP32 column sums are added in wave order through
// LDS and written as one partial row: partial[gridDim.y][cols].
__global__ __launch_bounds__(256) void gelu_bwd_kernel(const uint4* __restrict__ dy,
                                                       const uint4* __restrict__ x,
                                                       const uint4* __restrict__ bias,
                                                       uint4* __restrict__ dx,
                                                       float* __restrict__ partial, int64_t rows,
                                                       int vecs, int rows_per_wave, GeluConsts g) {
  __shared__ float red[3][kWave][8];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int v = blockIdx.x * kWave + lane;
  const bool active = v < vecs;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (active) {
    float bv[8];
    unpack8(bias[v], bv);
    const int64_t r0 = ((int64_t)blockIdx.y * 4 + wave) * rows_per_wave;
    const int64_t r1 = min(rows, r0 + rows_per_wave);
    for (int64_t r = r0; r < r1; r += kUnroll) {
      uint4 xv[kUnroll], dv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (r + u < r1) {
          xv[u] = ld_nt(x + (r + u) * vecs + v);
          dv[u] = ld_nt(dy + (r + u) * vecs + v);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (r + u < r1) {
          float f[8], d[8], o[8];
          unpack8(xv[u], f);
          unpack8(dv[u], d);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float uu = f[e] + bv[e];
            const float s = logistic_part(uu, g);
            const float grad = fmaf(g.k2 * uu * s * (1.0f - s), fmaf(g.c3, uu * uu, 1.0f), s);
            o[e] = d[e] * grad;
            acc[e] += o[e];
          }
          st_nt(dx + (r + u) * vecs + v, pack8(o));
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave - 1][lane][e] = acc[e];
  }
  __syncthreads();
  if (wave == 0 && active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = ((acc[e] + red[0][lane][e]) + red[1][lane][e]) + red[2][lane][e];
    const int64_t cols = (int64_t)vecs * 8;
    float4* out = reinterpret_cast<float4*>(partial + (int64_t)blockIdx.y * cols + (int64_t)v * 8);
    out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

GeluConsts gelu_consts() {
  GeluConsts g;
  g.a = (float)(-2.0 * kKd * kLog2e);
  g.b = (float)(-2.0 * kKd * kCd * kLog2e);
  g.k2 = (float)(2.0 * kKd);
  g.c3 = (float)(3.0 * kCd);
  return g;
}

struct GeluPlan {
  dim3 grid, block;
  int rows_per_block;
};

GeluPlan plan_gelu(int64_t rows, int vecs, int rows_per_block) {
  GeluPlan p;
  const int threads = vecs < 256 ? ((vecs + 63) / 64) * 64 : 256;
  p.block = dim3(threads);
  p.rows_per_block = rows_per_block;
  p.grid = dim3(ceil_div(vecs, threads), ceil_div(rows, rows_per_block));
  return p;
}

constexpr int kFwdRows = 8;
constexpr int kBwdRowsPerWave = 8;
constexpr int kBwdRows = 4 * kBwdRowsPerWave;  // rows per workgroup strip (one dbias partial row)

bloom_status check_gelu(int64_t rows, int64_t cols) {
  BLOOM_REQUIRE(rows >= 0, BLOOM_ERR_SHAPE, "rows = %lld is negative", (long long)rows);
  BLOOM_REQUIRE(cols >= 8 && cols <= BLOOM_MAX_HIDDEN && cols % 8 == 0, BLOOM_ERR_SHAPE,
                "cols = %lld must be a multiple of 8 in [8, %d]", (long long)cols,
                BLOOM_MAX_HIDDEN);
  BLOOM_REQUIRE(rows <= (int64_t)kFwdRows * 65535, BLOOM_ERR_SHAPE, "rows = %lld too large",
                (long long)rows);
  return BLOOM_OK;
}

}  // namespace
}  // namespace bloom

using namespace bloom;

extern "C" bloom_status bloom_bias_gelu_fwd(const bloom_bf16* x, const bloom_bf16* bias,
                                            bloom_bf16* y, int64_t rows, int64_t cols,
                                            hipStream_t stream) {
  clear_error();
  if (bloom_status st = check_gelu(rows, cols)) return st;
  if (rows == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(x);
  BLOOM_REQUIRE_PTR(bias);
  BLOOM_REQUIRE_PTR(y);
  const int vecs = (int)(cols / 8);
  const GeluPlan p = plan_gelu(rows, vecs, kFwdRows);
  hipLaunchKernelGGL(gelu_fwd_kernel, p.grid, p.block, 0, stream,
                     reinterpret_cast<const uint4*>(x), reinterpret_cast<const uint4*>(bias),
                     reinterpret_cast<uint4*>(y), rows, vecs, p.rows_per_block, gelu_consts());
  return launch_status("bloom_bias_gelu_fwd");
}

extern "C" size_t bloom_bias_gelu_bwd_workspace_size(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 8 != 0 || cols > BLOOM_MAX_HIDDEN) return 0;
  return (size_t)ceil_div(rows, kBwdRows) * (size_t)cols * sizeof(float);
}

extern "C" bloom_status bloom_bias_gelu_bwd(const bloom_bf16* dy, const bloom_bf16* x,
                                            const bloom_bf16* bias, bloom_bf16* dx,
                                            bloom_bf16* dbias, void* workspace,
                                            size_t workspace_bytes, int64_t rows, int64_t cols,
                                            hipStream_t stream) {
  clear_error();
  if (bloom_status st = check_gelu(rows, cols)) return st;
  if (rows == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(dy);
  BLOOM_REQUIRE_PTR(x);
  BLOOM_REQUIRE_PTR(bias);
  BLOOM_REQUIRE_PTR(dx);
  BLOOM_REQUIRE_PTR(dbias);
  BLOOM_REQUIRE(workspace != nullptr, BLOOM_ERR_WORKSPACE, "workspace is NULL");
  BLOOM_REQUIRE(aligned16(workspace), BLOOM_ERR_ALIGN, "workspace is not 16-byte aligned");
  const int vecs = (int)(cols / 8);
  const dim3 grid(ceil_div(vecs, kWave), ceil_div(rows, kBwdRows));
  const size_t need = (size_t)grid.y * (size_t)cols * sizeof(float);
  BLOOM_REQUIRE(workspace_bytes >= need, BLOOM_ERR_WORKSPACE,
                "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  float* partial = static_cast<float*>(workspace);
  hipLaunchKernelGGL(gelu_bwd_kernel, grid, dim3(4 * kWave), 0, stream,
                     reinterpret_cast<const uint4*>(dy), reinterpret_cast<const uint4*>(x),
                     reinterpret_cast<const uint4*>(bias), reinterpret_cast<uint4*>(dx), partial,
                     rows, vecs, kBwdRowsPerWave, gelu_consts());
  if (bloom_status st = launch_status("bloom_bias_gelu_bwd")) return st;
  launch_colsum(partial, (int)grid.y, cols, cols, dbias, nullptr, stream);
  return launch_status("bloom_bias_gelu_bwd column sums");
}
