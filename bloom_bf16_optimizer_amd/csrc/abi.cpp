// ABI plumbing: version, status strings, the thread-local error message, the
// launch check and the cached device query.  Also two host-only functions:
// the ALiBi slope table (the slope rule of the ALiBi paper, arXiv:2108.12409,
// cited by page "BLOOM 176B 训练技术概览" under "资源" for the bias of
// "架构微调") and the warmup + cosine learning-rate schedule of section 3's
// training config on page "单机多卡实战：Megatron-DeepSpeed训练类BLOOM模型全流程解析".
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "host_common.h"

namespace bloom {

namespace {
thread_local char g_error[512] = "";
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
}  // namespace

bloom_status fail(bloom_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_error[0] = '\0'; }

bloom_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BLOOM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return BLOOM_OK;
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace bloom

extern "C" {

int bloom_abi_version(void) { return 8; }

const char* bloom_status_string(int status) {
  switch (status) {
    case BLOOM_OK: return "ok";
    case BLOOM_ERR_NULL: return "null pointer";
    case BLOOM_ERR_SHAPE: return "invalid shape";
    case BLOOM_ERR_ALIGN: return "misaligned pointer";
    case BLOOM_ERR_WORKSPACE: return "workspace too small";
    case BLOOM_ERR_HPARAM: return "invalid scalar argument";
    case BLOOM_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bloom_last_error(void) { return bloom::g_error; }

bloom_status bloom_alibi_slopes(int32_t total_heads, int32_t head_offset, int32_t heads,
                                float* out_host) {
  bloom::clear_error();
  if (out_host == nullptr && heads > 0) return bloom::fail(BLOOM_ERR_NULL, "out_host is NULL");
  if (total_heads <= 0 || total_heads > (1 << 20) || head_offset < 0 || heads < 0 ||
      (int64_t)head_offset + heads > total_heads)
    return bloom::fail(BLOOM_ERR_SHAPE, "head range [%d, %d) outside a %d-head model", head_offset,
                       head_offset + heads, total_heads);
  // c = largest power of two <= total_heads.
  int32_t c = 1;
  while (c * 2 <= total_heads) c *= 2;
  for (int32_t k = 0; k < heads; ++k) {
    const int32_t h = head_offset + k;  // 0-based head index
    double e;                           // slope = 2^e
    if (h < c) {
      e = -8.0 * (double)(h + 1) / (double)c;  // power-of-two rule for c heads
    } else {
      // the (h-c)-th of the 1st, 3rd, 5th, ... slopes of the rule for 2c heads
      const int32_t j = 2 * (h - c) + 1;
      e = -8.0 * (double)j / (double)(2 * c);
    }
    out_host[k] = (float)std::exp2(e);
  }
  return BLOOM_OK;
}

}  // extern "C"

extern "C" bloom_status bloom_lr_warmup_cosine(int64_t step, double max_lr, double min_lr,
                                               int64_t warmup_steps, int64_t decay_steps, double* lr_out) {
  bloom::clear_error();
  if (lr_out == nullptr) return bloom::fail(BLOOM_ERR_NULL, "lr_out is NULL");
  if (step < 1) return bloom::fail(BLOOM_ERR_HPARAM, "step = %lld must be >= 1", (long long)step);
  if (!(std::isfinite(max_lr) && std::isfinite(min_lr) && min_lr >= 0.0 && min_lr <= max_lr))
    return bloom::fail(BLOOM_ERR_HPARAM, "need 0 <= min_lr <= max_lr, both finite");
  if (warmup_steps < 0 || decay_steps <= warmup_steps)
    return bloom::fail(BLOOM_ERR_HPARAM, "need 0 <= warmup_steps < decay_steps");
  const double pi = 3.14159265358979323846;
  if (warmup_steps > 0 && step <= warmup_steps) {
    *lr_out = max_lr * (double)step / (double)warmup_steps;
  } else if (step >= decay_steps) {
    *lr_out = min_lr;
  } else {
    const double q = (double)(step - warmup_steps) / (double)(decay_steps - warmup_steps);
    *lr_out = min_lr + (max_lr - min_lr) * 0.5 * (1.0 + std::cos(pi * q));
  }
  return BLOOM_OK;
}
