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
//   y'(u) = s + [u*(2k + 6kc u^2)] * [s(1-s)],
// evaluated as fma(p, q, s) with q = fma(-s, s, s) and p = u*fma(6kc, u^2, 2k)
// (u^2 is shared with the exponent).
//
// Mapping: a thread owns one 16-byte column vector (8 columns) for a strip of
// rows, keeping the 8 bias values -- and, in the backward, 8 FP32 dbias sums
// -- in registers.  Consecutive threads own consecutive vectors, so each wave
// reads and writes 1 KiB contiguous per row.  The backward writes one FP32
// partial row per row strip; colsum.hip adds them in strip order.
//
// Latency: a full strip issues all of its row loads before the first row is
// computed (straight-line code, no guards), so the compiler can wait for each
// row with a partial vmcnt; the backward runs its strip as a two-deep stage
// pipeline, the loads of stage k+2 in flight while stage k is computed.
#include "device_common.h"
#include "host_common.h"
#include "launch_plan.h"

namespace bloom {
namespace {

constexpr double kKd = 0.7978845608028654;
constexpr double kCd = 0.044715;
constexpr double kLog2e = 1.4426950408889634;
constexpr int kFwdRows = 2;                              // rows per forward strip
constexpr int kBwdStageRows = 2;                         // rows per backward stage
constexpr int kBwdStages = 4;                            // stages per wave
constexpr int kBwdRowsPerWave = kBwdStageRows * kBwdStages;
constexpr int kBwdRows = 4 * kBwdRowsPerWave;            // rows per workgroup strip (one dbias partial row)
// The backward reserves LDS it never touches so that at most two workgroups
// (eight waves) share a compute unit: 4 % faster at [2048, 14336] than the
// five its registers allow.
constexpr size_t kBwdCapLds = 48 * 1024;

struct GeluConsts {
  float a;     // -2k log2(e)
  float b;     // -2kc log2(e)
  float k2;    // 2k
  float k6c;   // 6kc
};

// s = 1/(1 + exp(-2a)) with the hardware exp2 and reciprocal (each within
// 1 ulp of fp32; exp2 results below 2^-126 flush to 0, which leaves s = 1).
// The element budget is tight: at 8 TB/s the forward has ~20 VALU slots per
// element, so the correctly rounded divide (about 10 instructions) is not used.
__device__ __forceinline__ float logistic_part(float u, float u2, const GeluConsts& g) {
  const float t = __builtin_amdgcn_exp2f(u * fmaf(g.b, u2, g.a));
  return __builtin_amdgcn_rcpf(1.0f + t);
}

__device__ __forceinline__ float gelu_value(float u, const GeluConsts& g) {
  return u * logistic_part(u, u * u, g);
}

__device__ __forceinline__ float gelu_slope(float u, const GeluConsts& g) {
  const float u2 = u * u;
  const float s = logistic_part(u, u2, g);
  const float q = fmaf(-s, s, s);             // s(1-s)
  const float p = u * fmaf(g.k6c, u2, g.k2);  // 2k u (1 + 3c u^2)
  return fmaf(p, q, s);
}

__device__ __forceinline__ uint4 gelu_row(const uint4& xv, const float (&bv)[8], const GeluConsts& g) {
  float f[8], o[8];
  unpack8(xv, f);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = gelu_value(f[e] + bv[e], g);
  return pack8(o);
}

__device__ __forceinline__ uint4 gelu_grad_row(const uint4& dv, const uint4& xv, const float (&bv)[8],
                                               float (&acc)[8], const GeluConsts& g) {
  float f[8], d[8], o[8];
  unpack8(xv, f);
  unpack8(dv, d);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    o[e] = d[e] * gelu_slope(f[e] + bv[e], g);
    acc[e] += o[e];
  }
  return pack8(o);
}

// Forward: a 1-D grid of (row strip, column block) pairs, column block
// fastest, so consecutive workgroups sweep whole rows of kFwdRows rows
// (contiguous memory) and the grid has no 65535 limit on the row strips.
__global__ __launch_bounds__(256) void gelu_fwd_kernel(const uint4* __restrict__ x,
                                                       const uint4* __restrict__ bias,
                                                       uint4* __restrict__ y, int64_t rows, int vecs,
                                                       int col_blocks, GeluConsts g) {
  const int cb = (int)(blockIdx.x % (unsigned)col_blocks);
  const int64_t strip = blockIdx.x / (unsigned)col_blocks;
  const int v = cb * blockDim.x + threadIdx.x;
  if (v >= vecs) return;
  float bv[8];
  unpack8(bias[v], bv);
  const int64_t r0 = strip * kFwdRows;
  if (r0 + kFwdRows <= rows) {
    uint4 xv[kFwdRows];
#pragma unroll
    for (int u = 0; u < kFwdRows; ++u) xv[u] = ld_nt(x + (r0 + u) * vecs + v);
#pragma unroll
    for (int u = 0; u < kFwdRows; ++u) st_nt(y + (r0 + u) * vecs + v, gelu_row(xv[u], bv, g));
  } else {
    for (int64_t r = r0; r < rows; ++r) st_nt(y + r * vecs + v, gelu_row(ld_nt(x + r * vecs + v), bv, g));
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
                                                       int vecs, GeluConsts g) {
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
    const int64_t r0 = ((int64_t)blockIdx.y * 4 + wave) * kBwdRowsPerWave;
    if (r0 + kBwdRowsPerWave <= rows) {
      // kBwdStages stages of kBwdStageRows rows; two stages of loads in flight.
      uint4 xv[2][kBwdStageRows], dv[2][kBwdStageRows];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < kBwdStageRows; ++u) {
          const int64_t r = r0 + st * kBwdStageRows + u;
          xv[st][u] = ld_nt(x + r * vecs + v);
          dv[st][u] = ld_nt(dy + r * vecs + v);
        }
#pragma unroll
      for (int st = 0; st < kBwdStages; ++st) {
        const int b = st & 1;
#pragma unroll
        for (int u = 0; u < kBwdStageRows; ++u) {
          const int64_t r = r0 + st * kBwdStageRows + u;
          st_nt(dx + r * vecs + v, gelu_grad_row(dv[b][u], xv[b][u], bv, acc, g));
        }
        if (st + 2 < kBwdStages) {
#pragma unroll
          for (int u = 0; u < kBwdStageRows; ++u) {
            const int64_t r = r0 + (st + 2) * kBwdStageRows + u;
            xv[b][u] = ld_nt(x + r * vecs + v);
            dv[b][u] = ld_nt(dy + r * vecs + v);
          }
        }
      }
    } else {
      for (int64_t r = r0; r < rows && r < r0 + kBwdRowsPerWave; ++r)
        st_nt(dx + r * vecs + v, gelu_grad_row(ld_nt(dy + r * vecs + v), ld_nt(x + r * vecs + v), bv, acc, g));
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
  g.k6c = (float)(6.0 * kKd * kCd);
  return g;
}

bloom_status check_gelu(int64_t rows, int64_t cols) {
  BLOOM_REQUIRE(rows >= 0, BLOOM_ERR_SHAPE, "rows = %lld is negative", (long long)rows);
  BLOOM_REQUIRE(cols >= 8 && cols <= BLOOM_MAX_HIDDEN && cols % 8 == 0, BLOOM_ERR_SHAPE,
                "cols = %lld must be a multiple of 8 in [8, %d]", (long long)cols,
                BLOOM_MAX_HIDDEN);
  BLOOM_REQUIRE(rows <= (int64_t)kBwdRows * 65535, BLOOM_ERR_SHAPE, "rows = %lld too large",
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
  const int threads = vecs < 256 ? ((vecs + 63) / 64) * 64 : 256;
  const int col_blocks = ceil_div(vecs, threads);
  const int64_t blocks = (int64_t)ceil_div(rows, kFwdRows) * col_blocks;
  BLOOM_REQUIRE(blocks <= 0x7fffffff, BLOOM_ERR_SHAPE, "rows = %lld too large", (long long)rows);
  hipLaunchKernelGGL(gelu_fwd_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     reinterpret_cast<const uint4*>(x), reinterpret_cast<const uint4*>(bias),
                     reinterpret_cast<uint4*>(y), rows, vecs, col_blocks, gelu_consts());
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
  hipLaunchKernelGGL(gelu_bwd_kernel, grid, dim3(4 * kWave), kBwdCapLds, stream,
                     reinterpret_cast<const uint4*>(dy), reinterpret_cast<const uint4*>(x),
                     reinterpret_cast<const uint4*>(bias), reinterpret_cast<uint4*>(dx), partial,
                     rows, vecs, gelu_consts());
  if (bloom_status st = launch_status("bloom_bias_gelu_bwd")) return st;
  launch_colsum(partial, (int)grid.y, cols, cols, dbias, nullptr, stream);
  return launch_status("bloom_bias_gelu_bwd column sums");
}
