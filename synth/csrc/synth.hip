// Device side of the seeded input generator: fills a tensor with the values
// synth/__init__.py defines, bit for bit (SplitMix64 counter draws, twelve
// 16-bit fields summed Irwin-Hall style, one fp32 multiply and an optional
// fp32 add).  Built with -ffp-contract=off so the multiply and add stay two
// separately rounded operations, as on the host.  Holds no arithmetic of the
// kernels it feeds.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr int kBlock = 256;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float value(uint64_t key, uint64_t idx, float scale, float offset,
                                       int add_offset) {
  int32_t s = 0;
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    const uint64_t u = mix64(key + (idx * 3ull + (uint64_t)d + 1ull) * kGamma);
    s += (int32_t)(u & 0xFFFFull) + (int32_t)((u >> 16) & 0xFFFFull) +
         (int32_t)((u >> 32) & 0xFFFFull) + (int32_t)(u >> 48);
  }
  float z = __fmul_rn((float)(s - 393210), scale);
  if (add_offset) z = __fadd_rn(z, offset);
  return z;
}

// mode 0: fp32, 1: bf16 (upper 16 bits), 2: |fp32|
__global__ __launch_bounds__(kBlock) void fill_kernel(void* out, int64_t n, int64_t start,
                                                      uint64_t key, float scale, float offset,
                                                      int add_offset, int mode) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float z = value(key, (uint64_t)(start + i), scale, offset, add_offset);
    if (mode == 1) {
      static_cast<uint16_t*>(out)[i] = (uint16_t)(__float_as_uint(z) >> 16);
    } else {
      static_cast<float*>(out)[i] = (mode == 2) ? fabsf(z) : z;
    }
  }
}

}  // namespace

extern "C" int synth_fill(void* out, int64_t n, int64_t start, uint64_t key, float scale,
                          float offset, int add_offset, int mode, hipStream_t stream) {
  if (n < 0 || start < 0 || mode < 0 || mode > 2) return 2;
  if (n == 0) return 0;
  if (out == nullptr) return 1;
  int64_t blocks = (n + kBlock - 1) / kBlock;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream, out, n, start,
                     key, scale, offset, add_offset, mode);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
