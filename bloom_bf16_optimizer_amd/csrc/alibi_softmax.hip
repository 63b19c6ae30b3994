// Scale + ALiBi bias + causal mask + softmax, forward and backward, for gfx950.
//
// What is computed: the combined scale/mask/softmax kernel of page
// "BLOOM 176B 训练技术概览", section "融合 CUDA 核", with the ALiBi linear
// bias of "架构微调" (slopes from the ALiBi paper listed under "资源"); page
// "企业官网建设流程全解析", section 4.3 runs it at 8192 tokens.  For query row i
// of head h:  z_j = scale*s_ij - slope_h*(i-j) for j <= i, y = softmax(z) over
// j <= i, y_j = +0 for j > i; backward ds_j = scale*y_j*(dy_j - sum_k y_k dy_k).
//
// Memory traffic is the floor the method allows: only the causal part
// (16-byte vectors that hold at least one column j <= i) is read, and every
// output element is written once.  The exponent is taken base 2: the host
// passes scale*log2(e) and slope_h*log2(e) (derived in FP64), so
// exp(z - max) = exp2(z2 - max2).  The bias is formed relative to the
// diagonal, slope2*(j - i), which keeps it small and exact where it matters.
//
// Load balance: row i reads i+1 keys, so the team -> row map interleaves
// short and long rows (k even -> i = k/2, k odd -> i = L-1-(k-1)/2) and every
// pair of consecutive teams does the same work.
#include <cmath>

#include "device_common.h"
#include "host_common.h"
#include "launch_plan.h"

namespace bloom {
namespace {

struct SlopeTable {
  float s[BLOOM_MAX_HEADS];  // slope_h * log2(e), fp32
};

__device__ __forceinline__ int paired_row(int k, int seq) {
  return (k & 1) ? seq - 1 - (k >> 1) : (k >> 1);
}

template <int NV, int MAXB>
__global__ __launch_bounds__(MAXB) void softmax_fwd_kernel(
    const uint4* __restrict__ scores, uint4* __restrict__ probs, int64_t rows_total, int seq,
    int vecs, int tpr, int heads, float scale2, SlopeTable slopes) {
  __shared__ float lds[kMaxWaves];
  const bool wave_rows = (tpr == kWave);
  const int t = wave_rows ? (int)(threadIdx.x & (kWave - 1)) : (int)threadIdx.x;
  const int64_t q = wave_rows ? (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave
                              : (int64_t)blockIdx.x;
  if (q >= rows_total) return;  // uniform over the team
  const int nwaves = blockDim.x / kWave;
  const int64_t bh = q / seq;
  const int i = paired_row((int)(q - bh * seq), seq);
  const float slope2 = slopes.s[bh % heads];
  const int64_t row = bh * seq + i;
  const uint4* src = scores + row * vecs;
  uint4* dst = probs + row * vecs;
  const int nlive = (i >> 3) + 1;  // vectors holding some column j <= i

  // Loads without per-lane branches: a vector past the causal window
  // (v >= nlive, so every column j = 8v+e > i) re-reads the row's first
  // vector -- the same cache line for all such lanes, no extra HBM bytes --
  // and is masked by j <= i; only a k whose vectors are all past the window
  // for the whole team is skipped (a team-uniform branch).  The NV loads are
  // all in flight before the first is used.
  uint4 raw[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    raw[k] = make_uint4(0u, 0u, 0u, 0u);
    if (k * tpr < nlive) raw[k] = ld_nt(src + (v < nlive ? v : 0));  // team-uniform test
  }
  float z[NV][8];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    float s[8];
    unpack8(raw[k], s);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = v * 8 + e;
      z[k][e] = (j <= i) ? fmaf(s[e], scale2, slope2 * (float)(j - i)) : -INFINITY;
      mx = fmaxf(mx, z[k][e]);
    }
  }
  mx = wave_rows ? wave_max(mx) : block_max(mx, lds, nwaves);

  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // hardware exp2: exp2(-inf) = 0 for masked entries; results below
      // 2^-126 (probabilities under 1.2e-38) flush to 0.
      z[k][e] = __builtin_amdgcn_exp2f(z[k][e] - mx);
      sum += z[k][e];
    }
  }
  sum = wave_rows ? wave_sum(sum) : block_sum(sum, lds, nwaves);
  const float inv = 1.0f / sum;

#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    if (v < vecs) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = z[k][e] * inv;  // masked: exp2(-inf) * inv = +0
      st_nt(dst + v, pack8(o));
    }
  }
}

template <int NV, int MAXB>
__global__ __launch_bounds__(MAXB) void softmax_bwd_kernel(
    const uint4* __restrict__ probs, const uint4* __restrict__ dprobs, uint4* __restrict__ dscores,
    int64_t rows_total, int seq, int vecs, int tpr, float scale) {
  __shared__ float lds[kMaxWaves];
  const bool wave_rows = (tpr == kWave);
  const int t = wave_rows ? (int)(threadIdx.x & (kWave - 1)) : (int)threadIdx.x;
  const int64_t q = wave_rows ? (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave
                              : (int64_t)blockIdx.x;
  if (q >= rows_total) return;
  const int nwaves = blockDim.x / kWave;
  const int64_t bh = q / seq;
  const int i = paired_row((int)(q - bh * seq), seq);
  const int64_t row = bh * seq + i;
  const uint4* ys = probs + row * vecs;
  const uint4* dys = dprobs + row * vecs;
  uint4* dst = dscores + row * vecs;
  const int nlive = (i >> 3) + 1;

  // Loads as in the forward: lanes past the causal window re-read vector 0
  // and are masked by j <= i.
  uint4 yv[NV], dv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    const int vv = v < nlive ? v : 0;
    yv[k] = make_uint4(0u, 0u, 0u, 0u);
    dv[k] = yv[k];
    if (k * tpr < nlive) {  // team-uniform test
      yv[k] = ld_nt(ys + vv);
      dv[k] = ld_nt(dys + vv);
    }
  }
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    float y[8], d[8];
    unpack8(yv[k], y);
    unpack8(dv[k], d);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (v * 8 + e <= i) dot = fmaf(y[e], d[e], dot);
  }
  dot = wave_rows ? wave_sum(dot) : block_sum(dot, lds, nwaves);

#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = t + k * tpr;
    if (v < vecs) {
      float y[8], d[8], o[8];
      unpack8(yv[k], y);
      unpack8(dv[k], d);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v * 8 + e <= i) ? scale * y[e] * (d[e] - dot) : 0.f;
      st_nt(dst + v, pack8(o));
    }
  }
}

bloom_status check_softmax(int64_t batch, int32_t heads, int64_t seq) {
  BLOOM_REQUIRE(batch >= 0 && heads >= 0, BLOOM_ERR_SHAPE, "batch and heads must be >= 0");
  BLOOM_REQUIRE(batch <= (int64_t(1) << 31), BLOOM_ERR_SHAPE, "batch too large");
  BLOOM_REQUIRE(heads <= BLOOM_MAX_HEADS, BLOOM_ERR_SHAPE, "heads = %d exceeds %d", heads,
                BLOOM_MAX_HEADS);
  BLOOM_REQUIRE(seq >= 8 && seq <= BLOOM_MAX_SEQ && seq % 8 == 0, BLOOM_ERR_SHAPE,
                "seq = %lld must be a multiple of 8 in [8, %d]", (long long)seq, BLOOM_MAX_SEQ);
  BLOOM_REQUIRE(batch * heads * seq <= 0x7fffffffLL, BLOOM_ERR_SHAPE,
                "batch*heads*seq = %lld rows exceeds 2^31-1", (long long)(batch * heads * seq));
  return BLOOM_OK;
}

RowPlan plan_softmax(int64_t rows_total, int vecs) { return plan_rows_fwd(rows_total, vecs); }

// With a wave per row (rows up to 4096 wide), the kernels reserve LDS they
// never touch so that fewer workgroups share a compute unit: at most 6 in the
// forward and 4 in the backward.  Fewer row streams in flight measured 3 %
// and 2 % faster at [1, 28, 2048, 2048] than the 8 the registers allow.
size_t cap_lds(const RowPlan& p, bool bwd) {
  if (p.tpr != kWave) return 0;
  return bwd ? 40 * 1024 : 24 * 1024;
}

}  // namespace
}  // namespace bloom

using namespace bloom;

extern "C" bloom_status bloom_alibi_softmax_fwd(const bloom_bf16* scores, bloom_bf16* probs,
                                                int64_t batch, int32_t heads, int64_t seq,
                                                int32_t head_offset, int32_t total_heads,
                                                float scale, hipStream_t stream) {
  clear_error();
  if (bloom_status st = check_softmax(batch, heads, seq)) return st;
  BLOOM_REQUIRE(std::isfinite(scale), BLOOM_ERR_HPARAM, "scale must be finite");
  BLOOM_REQUIRE(total_heads > 0 && head_offset >= 0 && (int64_t)head_offset + heads <= total_heads,
                BLOOM_ERR_SHAPE, "heads [%d, %d) outside a %d-head model", head_offset,
                head_offset + heads, total_heads);
  if (batch == 0 || heads == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(scores);
  BLOOM_REQUIRE_PTR(probs);
  float slopes[BLOOM_MAX_HEADS];
  if (bloom_status st = bloom_alibi_slopes(total_heads, head_offset, heads, slopes)) return st;
  SlopeTable table;
  const double log2e = 1.4426950408889634;
  for (int h = 0; h < BLOOM_MAX_HEADS; ++h)
    table.s[h] = (h < heads) ? (float)((double)slopes[h] * log2e) : 0.f;
  const float scale2 = (float)((double)scale * log2e);
  const int64_t rows_total = batch * heads * seq;
  const int vecs = (int)(seq / 8);
  const RowPlan p = plan_softmax(rows_total, vecs);
  const uint4* src = reinterpret_cast<const uint4*>(scores);
  uint4* dst = reinterpret_cast<uint4*>(probs);
#define CALL(NV, MAXB)                                                                   \
  hipLaunchKernelGGL((softmax_fwd_kernel<NV, MAXB>), dim3(p.grid), dim3(p.block), cap_lds(p, false), stream, \
                     src, dst, rows_total, (int)seq, vecs, p.tpr, (int)heads, scale2, table)
  BLOOM_ROW_DISPATCH(p, CALL);
#undef CALL
  return launch_status("bloom_alibi_softmax_fwd");
}

extern "C" bloom_status bloom_alibi_softmax_bwd(const bloom_bf16* probs, const bloom_bf16* dprobs,
                                                bloom_bf16* dscores, int64_t batch, int32_t heads,
                                                int64_t seq, float scale, hipStream_t stream) {
  clear_error();
  if (bloom_status st = check_softmax(batch, heads, seq)) return st;
  BLOOM_REQUIRE(std::isfinite(scale), BLOOM_ERR_HPARAM, "scale must be finite");
  if (batch == 0 || heads == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(probs);
  BLOOM_REQUIRE_PTR(dprobs);
  BLOOM_REQUIRE_PTR(dscores);
  const int64_t rows_total = batch * heads * seq;
  const int vecs = (int)(seq / 8);
  const RowPlan p = plan_softmax(rows_total, vecs);
  const uint4* ys = reinterpret_cast<const uint4*>(probs);
  const uint4* ds = reinterpret_cast<const uint4*>(dprobs);
  uint4* dst = reinterpret_cast<uint4*>(dscores);
#define CALL(NV, MAXB)                                                                   \
  hipLaunchKernelGGL((softmax_bwd_kernel<NV, MAXB>), dim3(p.grid), dim3(p.block), cap_lds(p, true), stream, \
                     ys, ds, dst, rows_total, (int)seq, vecs, p.tpr, scale)
  BLOOM_ROW_DISPATCH(p, CALL);
#undef CALL
  return launch_status("bloom_alibi_softmax_bwd");
}
