// Column sums of FP32 partial rows -> bf16, shared by the LayerNorm backward
// (dgamma, dbeta) and the bias-GeLU backward (dbias).
//
// A workgroup of 256 threads covers 64 columns: 16 column quads (float4) by
// 16 partial-row lanes.  Lane p adds rows p, p+16, p+32, ... in order; the 16
// lane totals are then added in lane order through LDS.  The order depends
// only on (parts, cols), so the result is deterministic.
#include "device_common.h"
#include "host_common.h"
#include "launch_plan.h"

namespace bloom {
namespace {

constexpr int kQuads = 16;
constexpr int kLanes = 16;
constexpr int kBatch = 8;

__global__ __launch_bounds__(kQuads* kLanes) void colsum_kernel(const float* __restrict__ partial,
                                                                int parts, int64_t cols,
                                                                int64_t split,
                                                                uint16_t* __restrict__ out0,
                                                                uint16_t* __restrict__ out1) {
  __shared__ float4 acc[kLanes][kQuads];
  const int q = threadIdx.x % kQuads;
  const int lane = threadIdx.x / kQuads;
  const int64_t c = ((int64_t)blockIdx.x * kQuads + q) * 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < cols) {
    // kBatch loads are issued before any of them is added, so a lane keeps
    // that many requests in flight; the additions still run in row order.
    for (int p0 = lane; p0 < parts; p0 += kLanes * kBatch) {
      float4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = p0 + u * kLanes;
        v[u] = (p < parts) ? *reinterpret_cast<const float4*>(partial + (int64_t)p * cols + c)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (p0 + u * kLanes < parts) {
          s.x += v[u].x;
          s.y += v[u].y;
          s.z += v[u].z;
          s.w += v[u].w;
        }
      }
    }
  }
  acc[lane][q] = s;
  __syncthreads();
  if (lane == 0 && c < cols) {
    float4 t = acc[0][q];
    for (int l = 1; l < kLanes; ++l) {
      const float4 v = acc[l][q];
      t.x += v.x;
      t.y += v.y;
      t.z += v.z;
      t.w += v.w;
    }
    // four consecutive columns never straddle `split` (both are multiples of 4)
    uint16_t* dst = (c < split) ? out0 + c : out1 + (c - split);
    const uint32_t lo = pack2(t.x, t.y);
    const uint32_t hi = pack2(t.z, t.w);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  }
}

}  // namespace

void launch_colsum(const float* partial, int parts, int64_t cols, int64_t split, bloom_bf16* out0,
                   bloom_bf16* out1, hipStream_t stream) {
  const int grid = ceil_div(cols, kQuads * 4);
  hipLaunchKernelGGL(colsum_kernel, dim3(grid), dim3(kQuads * kLanes), 0, stream, partial, parts,
                     cols, split, out0, out1);
}

}  // namespace bloom
