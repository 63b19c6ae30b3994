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
// Memory hints.  Every load and store of the streams is non-temporal: each
// element is touched once per pass and not again until tens of gigabytes of
// other traffic have gone by.
//
// Launch shape.  Every pass is a flat stream: one workgroup of 256 threads per
// 1024 consecutive elements, each thread one "quad" of 4 elements, so every
// wave-wide load or store instruction covers one contiguous span (512 B of
// bf16, 1 KiB of fp32).  Workgroup ids go round-robin over the 8 XCDs; the
// logical block is remapped so that each XCD sweeps one contiguous eighth of
// the arrays.  Indices are 64-bit (n reaches 3.67e9); a trailing partial quad
// is handled element by element.  Measured on MI355X this shape streams ~6
// TB/s where grid-stride loops with two 16-byte vectors per thread stay near 5.
//
// Norm.  Every workgroup writes the FP64 sum of acc^2 over its 1024 elements
// (exact float -> double widening, fused multiply-adds) to partials[logical
// block]; the partials are then added in a fixed order by a 2048-workgroup
// pass and a one-workgroup finalize that forms N and the clip coefficient c,
// which stay in device memory for the AdamW kernel (no host round trip).  The
// partials come either from a standalone read of acc or, with no extra
// traffic, from the last micro-batch's accumulation pass.  The per-block
// partials are identical either way, so both paths give the same bits.
#include <cmath>

#include "device_common.h"
#include "host_common.h"

namespace bloom {
namespace {

constexpr int kBlock = 256;              // threads per workgroup, one quad each
constexpr int64_t kBlockElems = 4 * kBlock;
constexpr int kStage2Blocks = 2048;      // second reduction level (8 sums per finalize thread)

// Occupancy cap for the passes with many concurrent streams (the multi
// micro-batch accumulation reads up to 17 arrays, AdamW reads 4 and writes 4):
// each workgroup reserves 31 KB of LDS it never touches, so at most 5
// workgroups (20 waves) share a CU.  Fewer requests in flight measured 1 %
// (accumulation of 8) and 4 % (AdamW) faster than 8 workgroups per CU at
// 3.67e9 elements, and 3 to 6 per CU within 0.3 % of each other for 8, 12 and
// 16 gradients; the one-gradient accumulation and the sum of squares measured
// slower with the cap and launch without it.
constexpr size_t kCapLds = 31 * 1024;

// Workgroups of a flat pass over n elements, rounded up to a multiple of 8 so
// that the XCD remap below is a permutation.
int64_t quad_blocks(int64_t n) {
  int64_t g = (n + kBlockElems - 1) / kBlockElems;
  if (g < 8) g = 8;
  return (g + 7) / 8 * 8;
}

// Logical block of this workgroup: block b runs on XCD b % 8; XCD x gets the
// contiguous logical range [x*G/8, (x+1)*G/8).
__device__ __forceinline__ int64_t xcd_block() {
  const int64_t b = blockIdx.x;
  const int64_t g = gridDim.x;
  return (b & 7) * (g >> 3) + (b >> 3);
}

// FP64 block sum (fixed order: shuffles in the wave, then waves in order).
__device__ __forceinline__ double block_sum_f64(double s) {
  __shared__ double lds[kBlock / kWave];
  s = wave_sum_f64(s);
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = s;
  __syncthreads();
  return (lds[0] + lds[1]) + (lds[2] + lds[3]);
}

// ---------------------------------------------------------------------------
// Stage 1: acc = float(g) (first micro-batch) or acc = acc + float(g); with
// SUMSQ also the block's FP64 sum of the new acc^2.
template <bool FIRST, bool SUMSQ>
__global__ __launch_bounds__(kBlock) void grad_accumulate_kernel(float* __restrict__ acc,
                                                                 const uint16_t* __restrict__ g,
                                                                 int64_t n,
                                                                 double* __restrict__ partial) {
  const int64_t lb = xcd_block();
  const int64_t q = lb * kBlock + threadIdx.x;
  const int64_t e0 = q * 4;
  double s = 0.0;
  if (e0 + 4 <= n) {
    const uint2 gv = ld_nt(reinterpret_cast<const uint2*>(g) + q);
    float4 r;
    if (FIRST) {
      r = make_float4(bf16_lo(gv.x), bf16_hi(gv.x), bf16_lo(gv.y), bf16_hi(gv.y));
    } else {
      r = ld_nt(reinterpret_cast<const float4*>(acc) + q);
      r.x += bf16_lo(gv.x);
      r.y += bf16_hi(gv.x);
      r.z += bf16_lo(gv.y);
      r.w += bf16_hi(gv.y);
    }
    st_nt(reinterpret_cast<float4*>(acc) + q, r);
    if (SUMSQ) {
      s = fma((double)r.x, (double)r.x, s);
      s = fma((double)r.y, (double)r.y, s);
      s = fma((double)r.z, (double)r.z, s);
      s = fma((double)r.w, (double)r.w, s);
    }
  } else if (e0 < n) {
    for (int64_t j = e0; j < n; ++j) {
      const float gf = __uint_as_float((uint32_t)g[j] << 16);
      const float r = FIRST ? gf : acc[j] + gf;
      acc[j] = r;
      if (SUMSQ) s = fma((double)r, (double)r, s);
    }
  }
  if (SUMSQ) {
    s = block_sum_f64(s);
    if (threadIdx.x == 0) partial[lb] = s;
  }
}

// Stage 1 over K micro-batches in one pass: acc = (((acc or float(g_0)) +
// float(g_1)) + ...) + float(g_{K-1}), the same FP32 additions in the same
// order as K single-micro-batch passes, with the accumulator read and written
// once.  All K gradient loads are issued before the first addition.
struct GradPtrs {
  const uint16_t* g[BLOOM_MAX_ACCUM_BATCH];
};

template <int K, bool FIRST, bool SUMSQ>
__global__ __launch_bounds__(kBlock) void grad_accumulate_many_kernel(float* __restrict__ acc, GradPtrs gp,
                                                                      int64_t n, double* __restrict__ partial) {
  const int64_t lb = xcd_block();
  const int64_t q = lb * kBlock + threadIdx.x;
  const int64_t e0 = q * 4;
  double s = 0.0;
  if (e0 + 4 <= n) {
    uint2 gv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) gv[k] = ld_nt(reinterpret_cast<const uint2*>(gp.g[k]) + q);
    float4 r;
    if (FIRST) {
      r = make_float4(bf16_lo(gv[0].x), bf16_hi(gv[0].x), bf16_lo(gv[0].y), bf16_hi(gv[0].y));
    } else {
      r = ld_nt(reinterpret_cast<const float4*>(acc) + q);
      r.x += bf16_lo(gv[0].x);
      r.y += bf16_hi(gv[0].x);
      r.z += bf16_lo(gv[0].y);
      r.w += bf16_hi(gv[0].y);
    }
#pragma unroll
    for (int k = 1; k < K; ++k) {
      r.x += bf16_lo(gv[k].x);
      r.y += bf16_hi(gv[k].x);
      r.z += bf16_lo(gv[k].y);
      r.w += bf16_hi(gv[k].y);
    }
    st_nt(reinterpret_cast<float4*>(acc) + q, r);
    if (SUMSQ) {
      s = fma((double)r.x, (double)r.x, s);
      s = fma((double)r.y, (double)r.y, s);
      s = fma((double)r.z, (double)r.z, s);
      s = fma((double)r.w, (double)r.w, s);
    }
  } else if (e0 < n) {
    for (int64_t j = e0; j < n; ++j) {
      const float g0 = __uint_as_float((uint32_t)gp.g[0][j] << 16);
      float r = FIRST ? g0 : acc[j] + g0;
#pragma unroll
      for (int k = 1; k < K; ++k) r += __uint_as_float((uint32_t)gp.g[k][j] << 16);
      acc[j] = r;
      if (SUMSQ) s = fma((double)r, (double)r, s);
    }
  }
  if (SUMSQ) {
    s = block_sum_f64(s);
    if (threadIdx.x == 0) partial[lb] = s;
  }
}

// Stage 2a (standalone): the same per-block partials from a read of acc.
__global__ __launch_bounds__(kBlock) void sumsq_kernel(const float* __restrict__ acc, int64_t n,
                                                       double* __restrict__ partial) {
  const int64_t lb = xcd_block();
  const int64_t q = lb * kBlock + threadIdx.x;
  const int64_t e0 = q * 4;
  double s = 0.0;
  if (e0 + 4 <= n) {
    const float4 r = ld_nt(reinterpret_cast<const float4*>(acc) + q);
    s = fma((double)r.x, (double)r.x, s);
    s = fma((double)r.y, (double)r.y, s);
    s = fma((double)r.z, (double)r.z, s);
    s = fma((double)r.w, (double)r.w, s);
  } else if (e0 < n) {
    for (int64_t j = e0; j < n; ++j) s = fma((double)acc[j], (double)acc[j], s);
  }
  s = block_sum_f64(s);
  if (threadIdx.x == 0) partial[lb] = s;
}

// Stage 2b: workgroup j adds partials [j*chunk, (j+1)*chunk) in a fixed order.
__global__ __launch_bounds__(kBlock) void partial_reduce_kernel(const double* __restrict__ partial,
                                                                int64_t parts, int64_t chunk,
                                                                double* __restrict__ out) {
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  int64_t hi = lo + chunk;
  if (hi > parts) hi = parts;
  double s = 0.0;
  for (int64_t p = lo + threadIdx.x; p < hi; p += kBlock) s += partial[p];
  s = block_sum_f64(s);
  if (threadIdx.x == 0) out[blockIdx.x] = s;
}

struct NormState {
  double sumsq;
  double norm;
  float clip;  // read by the AdamW kernel
  float pad[3];
};

// Stage 2c: one workgroup adds the stage-2 sums in order, forms N and c.
__global__ __launch_bounds__(kBlock) void norm_finalize_kernel(const double* __restrict__ part2,
                                                               double max_norm,
                                                               NormState* __restrict__ state,
                                                               float* __restrict__ norm_out) {
  double s = 0.0;
  for (int k = 0; k < kStage2Blocks / kBlock; ++k) s += part2[threadIdx.x * (kStage2Blocks / kBlock) + k];
  const double t = block_sum_f64(s);
  if (threadIdx.x == 0) {
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
  const int64_t q = xcd_block() * kBlock + threadIdx.x;
  const int64_t e0 = q * 4;
  if (e0 + 4 <= n) {
    const float4 a = ld_nt(reinterpret_cast<const float4*>(acc) + q);
    float4 p = ld_nt(reinterpret_cast<const float4*>(master) + q);
    float4 m = ld_nt(reinterpret_cast<const float4*>(exp_avg) + q);
    float4 v = ld_nt(reinterpret_cast<const float4*>(exp_avg_sq) + q);
    adam_one(a.x, c, p.x, m.x, v.x, k);
    adam_one(a.y, c, p.y, m.y, v.y, k);
    adam_one(a.z, c, p.z, m.z, v.z, k);
    adam_one(a.w, c, p.w, m.w, v.w, k);
    st_nt(reinterpret_cast<float4*>(master) + q, p);
    st_nt(reinterpret_cast<float4*>(exp_avg) + q, m);
    st_nt(reinterpret_cast<float4*>(exp_avg_sq) + q, v);
    st_nt(reinterpret_cast<uint2*>(param) + q, make_uint2(pack2(p.x, p.y), pack2(p.z, p.w)));
  } else if (e0 < n) {
    for (int64_t j = e0; j < n; ++j) {
      float p = master[j], m = exp_avg[j], v = exp_avg_sq[j];
      adam_one(acc[j], c, p, m, v, k);
      master[j] = p;
      exp_avg[j] = m;
      exp_avg_sq[j] = v;
      param[j] = (uint16_t)(pack2(p, 0.f) & 0xffffu);
    }
  }
}

// ---------------------------------------------------------------------------
// Workspace: [partials: quad_blocks(n) doubles][stage 2: 256 doubles][NormState],
// each part 256-byte aligned.
struct WorkspaceLayout {
  size_t partial_off, stage2_off, state_off, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

WorkspaceLayout workspace_layout(int64_t n) {
  WorkspaceLayout w;
  w.partial_off = 0;
  w.stage2_off = align256((size_t)quad_blocks(n) * sizeof(double));
  w.state_off = w.stage2_off + align256(kStage2Blocks * sizeof(double));
  w.total = w.state_off + align256(sizeof(NormState));
  return w;
}

bool finite_nonneg(double x) { return std::isfinite(x) && x >= 0.0; }

bloom_status launch_accumulate(float* acc, const bloom_bf16* grad, int64_t n, int32_t first,
                               double* partial, hipStream_t stream) {
  const dim3 grid((unsigned)quad_blocks(n));
  if (partial == nullptr) {
    if (first)
      hipLaunchKernelGGL((grad_accumulate_kernel<true, false>), grid, dim3(kBlock), 0, stream, acc,
                         grad, n, partial);
    else
      hipLaunchKernelGGL((grad_accumulate_kernel<false, false>), grid, dim3(kBlock), 0, stream,
                         acc, grad, n, partial);
  } else {
    if (first)
      hipLaunchKernelGGL((grad_accumulate_kernel<true, true>), grid, dim3(kBlock), 0, stream, acc,
                         grad, n, partial);
    else
      hipLaunchKernelGGL((grad_accumulate_kernel<false, true>), grid, dim3(kBlock), 0, stream, acc,
                         grad, n, partial);
  }
  return launch_status("bloom_bf16_grad_accumulate");
}

template <int K>
void launch_accumulate_many_k(float* acc, const GradPtrs& gp, int64_t n, bool first, double* partial,
                              hipStream_t stream) {
  const dim3 grid((unsigned)quad_blocks(n));
  if (partial == nullptr) {
    if (first)
      hipLaunchKernelGGL((grad_accumulate_many_kernel<K, true, false>), grid, dim3(kBlock), kCapLds, stream, acc, gp,
                         n, partial);
    else
      hipLaunchKernelGGL((grad_accumulate_many_kernel<K, false, false>), grid, dim3(kBlock), kCapLds, stream, acc, gp,
                         n, partial);
  } else {
    if (first)
      hipLaunchKernelGGL((grad_accumulate_many_kernel<K, true, true>), grid, dim3(kBlock), kCapLds, stream, acc, gp, n,
                         partial);
    else
      hipLaunchKernelGGL((grad_accumulate_many_kernel<K, false, true>), grid, dim3(kBlock), kCapLds, stream, acc, gp,
                         n, partial);
  }
}

bloom_status launch_accumulate_many(float* acc, const GradPtrs& gp, int count, int64_t n, bool first,
                                    double* partial, hipStream_t stream) {
  switch (count) {
    case 1: launch_accumulate_many_k<1>(acc, gp, n, first, partial, stream); break;
    case 2: launch_accumulate_many_k<2>(acc, gp, n, first, partial, stream); break;
    case 3: launch_accumulate_many_k<3>(acc, gp, n, first, partial, stream); break;
    case 4: launch_accumulate_many_k<4>(acc, gp, n, first, partial, stream); break;
    case 5: launch_accumulate_many_k<5>(acc, gp, n, first, partial, stream); break;
    case 6: launch_accumulate_many_k<6>(acc, gp, n, first, partial, stream); break;
    case 7: launch_accumulate_many_k<7>(acc, gp, n, first, partial, stream); break;
    case 8: launch_accumulate_many_k<8>(acc, gp, n, first, partial, stream); break;
    case 9: launch_accumulate_many_k<9>(acc, gp, n, first, partial, stream); break;
    case 10: launch_accumulate_many_k<10>(acc, gp, n, first, partial, stream); break;
    case 11: launch_accumulate_many_k<11>(acc, gp, n, first, partial, stream); break;
    case 12: launch_accumulate_many_k<12>(acc, gp, n, first, partial, stream); break;
    case 13: launch_accumulate_many_k<13>(acc, gp, n, first, partial, stream); break;
    case 14: launch_accumulate_many_k<14>(acc, gp, n, first, partial, stream); break;
    case 15: launch_accumulate_many_k<15>(acc, gp, n, first, partial, stream); break;
    default: launch_accumulate_many_k<16>(acc, gp, n, first, partial, stream); break;
  }
  return launch_status("bloom_bf16_grad_accumulate_many");
}
static_assert(BLOOM_MAX_ACCUM_BATCH == 16, "launch_accumulate_many covers 1..16 micro-batches");

// Largest n: quad_blocks(n) must fit a 32-bit grid.
constexpr int64_t kMaxElems = (int64_t)0x7ffffff0 * kBlockElems;

}  // namespace
}  // namespace bloom

using namespace bloom;

extern "C" bloom_status bloom_bf16_grad_accumulate(float* grad_acc, const bloom_bf16* grad,
                                                   int64_t n, int32_t first_microbatch,
                                                   hipStream_t stream) {
  clear_error();
  BLOOM_REQUIRE(n >= 0 && n <= kMaxElems, BLOOM_ERR_SHAPE, "n = %lld out of range", (long long)n);
  if (n == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(grad_acc);
  BLOOM_REQUIRE_PTR(grad);
  return launch_accumulate(grad_acc, grad, n, first_microbatch, nullptr, stream);
}

extern "C" size_t bloom_bf16_adamw_workspace_size(int64_t n) {
  if (n < 0 || n > kMaxElems) return 0;
  return workspace_layout(n).total;
}

extern "C" bloom_status bloom_bf16_grad_accumulate_sumsq(float* grad_acc, const bloom_bf16* grad,
                                                         int64_t n, int32_t first_microbatch,
                                                         void* workspace, size_t workspace_bytes,
                                                         hipStream_t stream) {
  clear_error();
  BLOOM_REQUIRE(n >= 0 && n <= kMaxElems, BLOOM_ERR_SHAPE, "n = %lld out of range", (long long)n);
  if (n == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(grad_acc);
  BLOOM_REQUIRE_PTR(grad);
  BLOOM_REQUIRE(workspace != nullptr, BLOOM_ERR_WORKSPACE, "workspace is NULL");
  BLOOM_REQUIRE(aligned16(workspace), BLOOM_ERR_ALIGN, "workspace is not 16-byte aligned");
  const WorkspaceLayout w = workspace_layout(n);
  BLOOM_REQUIRE(workspace_bytes >= w.total, BLOOM_ERR_WORKSPACE,
                "workspace has %zu bytes, needs %zu", workspace_bytes, w.total);
  double* partial = reinterpret_cast<double*>(static_cast<char*>(workspace) + w.partial_off);
  return launch_accumulate(grad_acc, grad, n, first_microbatch, partial, stream);
}

extern "C" bloom_status bloom_bf16_grad_accumulate_many(float* grad_acc, const bloom_bf16* const* grads,
                                                        int32_t count, int64_t n, int32_t first_microbatch,
                                                        void* workspace, size_t workspace_bytes,
                                                        hipStream_t stream) {
  clear_error();
  BLOOM_REQUIRE(count >= 1 && count <= BLOOM_MAX_ACCUM_BATCH, BLOOM_ERR_SHAPE,
                "count = %d must be in [1, %d]", count, BLOOM_MAX_ACCUM_BATCH);
  BLOOM_REQUIRE(n >= 0 && n <= kMaxElems, BLOOM_ERR_SHAPE, "n = %lld out of range", (long long)n);
  if (n == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(grad_acc);
  BLOOM_REQUIRE(grads != nullptr, BLOOM_ERR_NULL, "grads is NULL");
  GradPtrs gp = {};
  for (int k = 0; k < count; ++k) {
    BLOOM_REQUIRE(grads[k] != nullptr, BLOOM_ERR_NULL, "grads[%d] is NULL", k);
    BLOOM_REQUIRE(aligned16(grads[k]), BLOOM_ERR_ALIGN, "grads[%d] is not 16-byte aligned", k);
    gp.g[k] = grads[k];
  }
  double* partial = nullptr;
  if (workspace != nullptr) {
    BLOOM_REQUIRE(aligned16(workspace), BLOOM_ERR_ALIGN, "workspace is not 16-byte aligned");
    const WorkspaceLayout w = workspace_layout(n);
    BLOOM_REQUIRE(workspace_bytes >= w.total, BLOOM_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
                  workspace_bytes, w.total);
    partial = reinterpret_cast<double*>(static_cast<char*>(workspace) + w.partial_off);
  }
  return launch_accumulate_many(grad_acc, gp, count, n, first_microbatch != 0, partial, stream);
}

namespace bloom {
namespace {

// Shared by the flat and the segmented step: validation, norm, clip, then one
// AdamW launch per segment with that segment's decay.
bloom_status adamw_step_impl(const char* name, float* master, float* exp_avg, float* exp_avg_sq,
                             bloom_bf16* param_bf16, const float* grad_acc, int64_t n,
                             const bloom_adamw_hparams* hp, const bloom_adamw_segment* segments,
                             int32_t num_segments, float* grad_norm_out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  BLOOM_REQUIRE(n >= 0 && n <= kMaxElems, BLOOM_ERR_SHAPE, "n = %lld out of range", (long long)n);
  BLOOM_REQUIRE(hp != nullptr, BLOOM_ERR_NULL, "hp is NULL");
  BLOOM_REQUIRE(finite_nonneg(hp->lr), BLOOM_ERR_HPARAM, "lr must be finite and >= 0");
  BLOOM_REQUIRE(hp->beta1 >= 0.0 && hp->beta1 < 1.0, BLOOM_ERR_HPARAM, "beta1 must be in [0, 1)");
  BLOOM_REQUIRE(hp->beta2 >= 0.0 && hp->beta2 < 1.0, BLOOM_ERR_HPARAM, "beta2 must be in [0, 1)");
  BLOOM_REQUIRE(std::isfinite(hp->eps) && hp->eps > 0.0, BLOOM_ERR_HPARAM,
                "eps must be finite and > 0");
  BLOOM_REQUIRE(hp->max_grad_norm > 0.0, BLOOM_ERR_HPARAM, "max_grad_norm must be > 0");
  BLOOM_REQUIRE(hp->step >= 1, BLOOM_ERR_HPARAM, "step must be >= 1");
  BLOOM_REQUIRE(hp->sumsq_in_workspace == 0 || hp->sumsq_in_workspace == 1, BLOOM_ERR_HPARAM,
                "sumsq_in_workspace must be 0 or 1");
  BLOOM_REQUIRE(hp->reserved == 0, BLOOM_ERR_HPARAM, "reserved must be 0");
  BLOOM_REQUIRE(segments != nullptr, BLOOM_ERR_NULL, "segments is NULL");
  BLOOM_REQUIRE(num_segments >= 1, BLOOM_ERR_SHAPE, "num_segments = %d must be >= 1", num_segments);
  int64_t end = 0;
  for (int32_t sgi = 0; sgi < num_segments; ++sgi) {
    const bloom_adamw_segment& sg = segments[sgi];
    BLOOM_REQUIRE(sg.offset == end, BLOOM_ERR_SHAPE, "segment %d starts at %lld, expected %lld", sgi,
                  (long long)sg.offset, (long long)end);
    BLOOM_REQUIRE(sg.offset % 8 == 0, BLOOM_ERR_ALIGN, "segment %d offset %lld is not a multiple of 8",
                  sgi, (long long)sg.offset);
    BLOOM_REQUIRE(sg.length >= 1 || (n == 0 && num_segments == 1), BLOOM_ERR_SHAPE,
                  "segment %d has length %lld", sgi, (long long)sg.length);
    BLOOM_REQUIRE(finite_nonneg(sg.weight_decay), BLOOM_ERR_HPARAM,
                  "segment %d weight_decay must be finite and >= 0", sgi);
    end += sg.length;
  }
  BLOOM_REQUIRE(end == n, BLOOM_ERR_SHAPE, "segments end at %lld, n = %lld", (long long)end, (long long)n);
  if (n == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(master);
  BLOOM_REQUIRE_PTR(exp_avg);
  BLOOM_REQUIRE_PTR(exp_avg_sq);
  BLOOM_REQUIRE_PTR(param_bf16);
  BLOOM_REQUIRE_PTR(grad_acc);
  BLOOM_REQUIRE(workspace != nullptr, BLOOM_ERR_WORKSPACE, "workspace is NULL");
  BLOOM_REQUIRE(aligned16(workspace), BLOOM_ERR_ALIGN, "workspace is not 16-byte aligned");
  const WorkspaceLayout w = workspace_layout(n);
  BLOOM_REQUIRE(workspace_bytes >= w.total, BLOOM_ERR_WORKSPACE,
                "workspace has %zu bytes, needs %zu", workspace_bytes, w.total);
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

  char* ws = static_cast<char*>(workspace);
  double* partial = reinterpret_cast<double*>(ws + w.partial_off);
  double* stage2 = reinterpret_cast<double*>(ws + w.stage2_off);
  NormState* state = reinterpret_cast<NormState*>(ws + w.state_off);
  const int64_t parts = quad_blocks(n);
  if (!hp->sumsq_in_workspace) {
    hipLaunchKernelGGL(sumsq_kernel, dim3((unsigned)parts), dim3(kBlock), 0, stream, grad_acc, n,
                       partial);
    if (bloom_status st = launch_status(name)) return st;
  }
  const int64_t chunk = (parts + kStage2Blocks - 1) / kStage2Blocks;
  hipLaunchKernelGGL(partial_reduce_kernel, dim3(kStage2Blocks), dim3(kBlock), 0, stream, partial,
                     parts, chunk, stage2);
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(1), dim3(kBlock), 0, stream, stage2,
                     hp->max_grad_norm, state, grad_norm_out);
  if (bloom_status st = launch_status(name)) return st;
  for (int32_t sgi = 0; sgi < num_segments; ++sgi) {
    const bloom_adamw_segment& sg = segments[sgi];
    k.lr_wd = (float)(hp->lr * sg.weight_decay);
    const int64_t o = sg.offset;
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)quad_blocks(sg.length)), dim3(kBlock), kCapLds, stream,
                       master + o, exp_avg + o, exp_avg_sq + o, param_bf16 + o, grad_acc + o, sg.length,
                       state, k);
    if (bloom_status st = launch_status(name)) return st;
  }
  return BLOOM_OK;
}

}  // namespace
}  // namespace bloom

extern "C" bloom_status bloom_bf16_adamw_step(float* master, float* exp_avg, float* exp_avg_sq,
                                              bloom_bf16* param_bf16, const float* grad_acc,
                                              int64_t n, const bloom_adamw_hparams* hp,
                                              float* grad_norm_out, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  BLOOM_REQUIRE(hp != nullptr, BLOOM_ERR_NULL, "hp is NULL");
  BLOOM_REQUIRE(finite_nonneg(hp->weight_decay), BLOOM_ERR_HPARAM,
                "weight_decay must be finite and >= 0");
  const bloom_adamw_segment all = {0, n, hp->weight_decay};
  return adamw_step_impl("bloom_bf16_adamw_step", master, exp_avg, exp_avg_sq, param_bf16, grad_acc, n, hp,
                         &all, 1, grad_norm_out, workspace, workspace_bytes, stream);
}

extern "C" bloom_status bloom_bf16_adamw_step_segments(float* master, float* exp_avg, float* exp_avg_sq,
                                                       bloom_bf16* param_bf16, const float* grad_acc,
                                                       int64_t n, const bloom_adamw_hparams* hp,
                                                       const bloom_adamw_segment* segments,
                                                       int32_t num_segments, float* grad_norm_out,
                                                       void* workspace, size_t workspace_bytes,
                                                       hipStream_t stream) {
  clear_error();
  return adamw_step_impl("bloom_bf16_adamw_step_segments", master, exp_avg, exp_avg_sq, param_bf16, grad_acc,
                         n, hp, segments, num_segments, grad_norm_out, workspace, workspace_bytes, stream);
}
