// BF16Optimizer for gfx950: FP32 gradient accumulation across micro-batches,
// global L2 norm and clip coefficient, AdamW on FP32 master weights and
// moments, and the round-to-nearest-even bf16 parameter copy.
//
// What is computed: page "BLOOM 176B 训练技术概览", section "BF16 优化器" (bf16
// mixed precision, all accumulation in FP32, FP32 gradient accumulation over
// the pipeline micro-batches); page "企业官网建设流程全解析", section 1 (FP32
// master parameters, momentum and variance), section 3.3 (32 accumulation
// steps, AdamW with lr 6e-5 and weight decay 0.01), section 4.3 (gradients
// clipped at global norm 1.0); page "单机多卡实战：Megatron-DeepSpeed训练类BLOOM
// 模型全流程解析", section 3 (the same lr, weight decay, clip and bf16 flags).
//
// All passes are flat, elementwise streams over n elements: 16-byte bf16
// vectors (8 elements) against pairs of 16-byte fp32 vectors, grid-stride
// loops with kUnroll groups of loads issued before any store, 64-bit indices
// (n reaches 3.67e9), and an n % 8 tail handled by the first threads.
//
// The norm is summed in FP64 (per-thread fused multiply-adds over exact
// float -> double widenings, four interleaved accumulators), reduced per
// workgroup, and the workgroup partials are added in workgroup order by a
// one-workgroup finalize kernel that also forms the clip coefficient.  The
// coefficient stays in device memory; the AdamW kernel reads it, so the step
// has no host round trip.
#include <cmath>

#include "device_common.h"
#include "host_common.h"

namespace bloom {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 2;
constexpr int kNormBlocksPerCu = 8;

// ---------------------------------------------------------------------------
// Stage 1: acc = float(g) (first micro-batch) or acc = acc + float(g).
template <bool FIRST>
__global__ __launch_bounds__(kBlock) void grad_accumulate_kernel(float* __restrict__ acc,
                                                                 const uint16_t* __restrict__ g,
                                                                 int64_t n) {
  const int64_t nvec = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const uint4* gv = reinterpret_cast<const uint4*>(g);
  float4* av = reinterpret_cast<float4*>(acc);
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; base < nvec;
       base += stride * kUnroll) {
    uint4 gr[kUnroll];
    float4 a0[kUnroll], a1[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * stride;
      if (i < nvec) {
        gr[u] = gv[i];
        if (!FIRST) {
          a0[u] = av[2 * i];
          a1[u] = av[2 * i + 1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * stride;
      if (i < nvec) {
        float f[8];
        unpack8(gr[u], f);
        if (FIRST) {
          av[2 * i] = make_float4(f[0], f[1], f[2], f[3]);
          av[2 * i + 1] = make_float4(f[4], f[5], f[6], f[7]);
        } else {
          av[2 * i] = make_float4(a0[u].x + f[0], a0[u].y + f[1], a0[u].z + f[2], a0[u].w + f[3]);
          av[2 * i + 1] =
              make_float4(a1[u].x + f[4], a1[u].y + f[5], a1[u].z + f[6], a1[u].w + f[7]);
        }
      }
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t j = (nvec << 3) + threadIdx.x;
    const float gf = __uint_as_float((uint32_t)g[j] << 16);
    acc[j] = FIRST ? gf : acc[j] + gf;
  }
}

// ---------------------------------------------------------------------------
// Stage 2a: per-workgroup FP64 partial sums of acc^2.
__global__ __launch_bounds__(kBlock) void sumsq_kernel(const float* __restrict__ acc, int64_t n,
                                                       double* __restrict__ partial) {
  __shared__ double lds[kBlock / kWave];
  const int64_t nvec = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const float4* av = reinterpret_cast<const float4*>(acc);
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; base < nvec;
       base += stride * 4) {
    float4 a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + u * stride;
      a[u] = (i < nvec) ? av[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s0 = fma((double)a[u].x, (double)a[u].x, s0);
      s1 = fma((double)a[u].y, (double)a[u].y, s1);
      s2 = fma((double)a[u].z, (double)a[u].z, s2);
      s3 = fma((double)a[u].w, (double)a[u].w, s3);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const double t = (double)acc[(nvec << 2) + threadIdx.x];
    s0 = fma(t, t, s0);
  }
  double s = wave_sum_f64((s0 + s1) + (s2 + s3));
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double b = 0.0;
    for (int w = 0; w < kBlock / kWave; ++w) b += lds[w];
    partial[blockIdx.x] = b;
  }
}

struct NormState {
  double sumsq;
  double norm;
  float clip;  // read by the AdamW kernel
  float pad[3];
};

// Stage 2b: one workgroup adds the partials in order, forms N and c.
__global__ __launch_bounds__(kBlock) void norm_finalize_kernel(const double* __restrict__ partial,
                                                               int parts, double max_norm,
                                                               NormState* __restrict__ state,
                                                               float* __restrict__ norm_out) {
  __shared__ double lds[kBlock];
  double s = 0.0;
  for (int p = threadIdx.x; p < parts; p += kBlock) s += partial[p];
  lds[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int k = 0; k < kBlock; ++k) t += lds[k];
    const double nrm = sqrt(t);
    // NaN compares false and leaves c = 1; an infinite norm gives c = 0.
    const double c = (nrm > max_norm) ? max_norm / nrm : 1.0;
    state->sumsq = t;
    state->norm = nrm;
    state->clip = (float)c;
    if (norm_out != nullptr) *norm_out = (float)nrm;
  }
}

// ---------------------------------------------------------------------------
// Stages 3-5: AdamW and the bf16 copy, one pass.
struct AdamConsts {
  float beta1, one_minus_beta1;
  float beta2, one_minus_beta2;
  float step_size;     // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
  float eps;
  float lr_wd;         // lr * weight_decay
};

__device__ __forceinline__ void adam_one(float a, float c, float& p, float& m, float& v,
                                         const AdamConsts& k) {
  const float g = c * a;
  m = fmaf(k.beta1, m, k.one_minus_beta1 * g);
  v = fmaf(k.beta2, v, k.one_minus_beta2 * (g * g));
  const float denom = fmaf(sqrtf(v), k.inv_sqrt_bc2, k.eps);
  p = p - k.step_size * (m / denom) - k.lr_wd * p;
}

__global__ __launch_bounds__(kBlock) void adamw_kernel(float* __restrict__ master,
                                                       float* __restrict__ exp_avg,
                                                       float* __restrict__ exp_avg_sq,
                                                       uint16_t* __restrict__ param,
                                                       const float* __restrict__ acc, int64_t n,
                                                       const NormState* __restrict__ state,
                                                       AdamConsts k) {
  const float c = state->clip;
  const int64_t nvec = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const float4* av = reinterpret_cast<const float4*>(acc);
  float4* pv = reinterpret_cast<float4*>(master);
  float4* mv = reinterpret_cast<float4*>(exp_avg);
  float4* vv = reinterpret_cast<float4*>(exp_avg_sq);
  uint4* ov = reinterpret_cast<uint4*>(param);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    float a[8], p[8], m[8], v[8];
    *reinterpret_cast<float4*>(a) = av[2 * i];
    *reinterpret_cast<float4*>(a + 4) = av[2 * i + 1];
    *reinterpret_cast<float4*>(p) = pv[2 * i];
    *reinterpret_cast<float4*>(p + 4) = pv[2 * i + 1];
    *reinterpret_cast<float4*>(m) = mv[2 * i];
    *reinterpret_cast<float4*>(m + 4) = mv[2 * i + 1];
    *reinterpret_cast<float4*>(v) = vv[2 * i];
    *reinterpret_cast<float4*>(v + 4) = vv[2 * i + 1];
#pragma unroll
    for (int e = 0; e < 8; ++e) adam_one(a[e], c, p[e], m[e], v[e], k);
    pv[2 * i] = *reinterpret_cast<float4*>(p);
    pv[2 * i + 1] = *reinterpret_cast<float4*>(p + 4);
    mv[2 * i] = *reinterpret_cast<float4*>(m);
    mv[2 * i + 1] = *reinterpret_cast<float4*>(m + 4);
    vv[2 * i] = *reinterpret_cast<float4*>(v);
    vv[2 * i + 1] = *reinterpret_cast<float4*>(v + 4);
    ov[i] = pack8(p);
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t j = (nvec << 3) + threadIdx.x;
    float p = master[j], m = exp_avg[j], v = exp_avg_sq[j];
    adam_one(acc[j], c, p, m, v, k);
    master[j] = p;
    exp_avg[j] = m;
    exp_avg_sq[j] = v;
    param[j] = (uint16_t)(pack2(p, 0.f) & 0xffffu);
  }
}

// ---------------------------------------------------------------------------
int stream_grid(int64_t nvec, int blocks_per_cu) {
  const int64_t cap = (int64_t)device_cu_count() * blocks_per_cu;
  int64_t need = (nvec + kBlock - 1) / kBlock;
  if (need < 1) need = 1;
  return (int)(need < cap ? need : cap);
}

int norm_parts(int64_t n) {
  const int64_t nvec = n >> 2;
  const int64_t cap = (int64_t)device_cu_count() * kNormBlocksPerCu;
  int64_t need = (nvec + kBlock - 1) / kBlock;
  if (need < 1) need = 1;
  return (int)(need < cap ? need : cap);
}

size_t adamw_workspace_bytes(int64_t n) {
  return (size_t)norm_parts(n) * sizeof(double) + sizeof(NormState) + 256;
}

bool finite_nonneg(double x) { return std::isfinite(x) && x >= 0.0; }

}  // namespace
}  // namespace bloom

using namespace bloom;

extern "C" bloom_status bloom_bf16_grad_accumulate(float* grad_acc, const bloom_bf16* grad,
                                                   int64_t n, int32_t first_microbatch,
                                                   hipStream_t stream) {
  clear_error();
  BLOOM_REQUIRE(n >= 0, BLOOM_ERR_SHAPE, "n = %lld is negative", (long long)n);
  if (n == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(grad_acc);
  BLOOM_REQUIRE_PTR(grad);
  const int grid = stream_grid(n >> 3, 8);
  if (first_microbatch)
    hipLaunchKernelGGL(grad_accumulate_kernel<true>, dim3(grid), dim3(kBlock), 0, stream, grad_acc,
                       grad, n);
  else
    hipLaunchKernelGGL(grad_accumulate_kernel<false>, dim3(grid), dim3(kBlock), 0, stream,
                       grad_acc, grad, n);
  return launch_status("bloom_bf16_grad_accumulate");
}

extern "C" size_t bloom_bf16_adamw_workspace_size(int64_t n) {
  if (n < 0) return 0;
  return adamw_workspace_bytes(n);
}

extern "C" bloom_status bloom_bf16_adamw_step(float* master, float* exp_avg, float* exp_avg_sq,
                                              bloom_bf16* param_bf16, const float* grad_acc,
                                              int64_t n, const bloom_adamw_hparams* hp,
                                              float* grad_norm_out, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  BLOOM_REQUIRE(n >= 0, BLOOM_ERR_SHAPE, "n = %lld is negative", (long long)n);
  BLOOM_REQUIRE(hp != nullptr, BLOOM_ERR_NULL, "hp is NULL");
  BLOOM_REQUIRE(finite_nonneg(hp->lr), BLOOM_ERR_HPARAM, "lr must be finite and >= 0");
  BLOOM_REQUIRE(hp->beta1 >= 0.0 && hp->beta1 < 1.0, BLOOM_ERR_HPARAM, "beta1 must be in [0, 1)");
  BLOOM_REQUIRE(hp->beta2 >= 0.0 && hp->beta2 < 1.0, BLOOM_ERR_HPARAM, "beta2 must be in [0, 1)");
  BLOOM_REQUIRE(std::isfinite(hp->eps) && hp->eps > 0.0, BLOOM_ERR_HPARAM,
                "eps must be finite and > 0");
  BLOOM_REQUIRE(finite_nonneg(hp->weight_decay), BLOOM_ERR_HPARAM,
                "weight_decay must be finite and >= 0");
  BLOOM_REQUIRE(hp->max_grad_norm > 0.0, BLOOM_ERR_HPARAM, "max_grad_norm must be > 0");
  BLOOM_REQUIRE(hp->step >= 1, BLOOM_ERR_HPARAM, "step must be >= 1");
  if (n == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(master);
  BLOOM_REQUIRE_PTR(exp_avg);
  BLOOM_REQUIRE_PTR(exp_avg_sq);
  BLOOM_REQUIRE_PTR(param_bf16);
  BLOOM_REQUIRE_PTR(grad_acc);
  BLOOM_REQUIRE(workspace != nullptr, BLOOM_ERR_WORKSPACE, "workspace is NULL");
  BLOOM_REQUIRE(aligned16(workspace), BLOOM_ERR_ALIGN, "workspace is not 16-byte aligned");
  const size_t need = adamw_workspace_bytes(n);
  BLOOM_REQUIRE(workspace_bytes >= need, BLOOM_ERR_WORKSPACE,
                "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  BLOOM_REQUIRE(grad_norm_out == nullptr || (reinterpret_cast<uintptr_t>(grad_norm_out) & 3) == 0,
                BLOOM_ERR_ALIGN, "grad_norm_out is not 4-byte aligned");

  // Every FP32 constant is derived in FP64 and rounded once.
  const double bc1 = 1.0 - std::pow(hp->beta1, (double)hp->step);
  const double bc2 = 1.0 - std::pow(hp->beta2, (double)hp->step);
  AdamConsts k;
  k.beta1 = (float)hp->beta1;
  k.one_minus_beta1 = (float)(1.0 - hp->beta1);
  k.beta2 = (float)hp->beta2;
  k.one_minus_beta2 = (float)(1.0 - hp->beta2);
  k.step_size = (float)(hp->lr / bc1);
  k.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  k.eps = (float)hp->eps;
  k.lr_wd = (float)(hp->lr * hp->weight_decay);

  const int parts = norm_parts(n);
  double* partial = static_cast<double*>(workspace);
  NormState* state = reinterpret_cast<NormState*>(
      static_cast<char*>(workspace) + ((size_t)parts * sizeof(double) + 255) / 256 * 256);
  hipLaunchKernelGGL(sumsq_kernel, dim3(parts), dim3(kBlock), 0, stream, grad_acc, n, partial);
  if (bloom_status st = launch_status("bloom_bf16_adamw_step: norm")) return st;
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(1), dim3(kBlock), 0, stream, partial, parts,
                     hp->max_grad_norm, state, grad_norm_out);
  if (bloom_status st = launch_status("bloom_bf16_adamw_step: clip")) return st;
  const int grid = stream_grid(n >> 3, 8);
  hipLaunchKernelGGL(adamw_kernel, dim3(grid), dim3(kBlock), 0, stream, master, exp_avg,
                     exp_avg_sq, param_bf16, grad_acc, n, state, k);
  return launch_status("bloom_bf16_adamw_step: update");
}
