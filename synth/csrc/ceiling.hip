// A plain streaming copy, used only to measure the achievable HBM rate of a
// given read/write pattern (the "copy ceiling" a kernel's bandwidth is
// compared with).  It computes nothing of the method: every output vector is
// the XOR of the input vectors at the same index (one input: a copy).
//
// Shape: one 16-byte vector per thread, 256 threads per workgroup, one flat
// grid over the vectors, non-temporal loads and stores -- the access style of
// the kernels it is compared with.  NIN inputs and NOUT outputs of `vecs`
// vectors each.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBlock = 256;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int NIN, int NOUT>
__global__ __launch_bounds__(kBlock) void stream_copy_kernel(u32x4_t* __restrict__ out0, u32x4_t* __restrict__ out1,
                                                             const u32x4_t* __restrict__ in0,
                                                             const u32x4_t* __restrict__ in1, int64_t vecs) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= vecs) return;
  u32x4_t v = __builtin_nontemporal_load(in0 + i);
  if (NIN == 2) v ^= __builtin_nontemporal_load(in1 + i);
  __builtin_nontemporal_store(v, out0 + i);
  if (NOUT == 2) __builtin_nontemporal_store(v, out1 + i);
}

template <int NIN, int NOUT>
void launch(void* out0, void* out1, const void* in0, const void* in1, int64_t vecs, hipStream_t stream) {
  const int64_t blocks = (vecs + kBlock - 1) / kBlock;
  hipLaunchKernelGGL((stream_copy_kernel<NIN, NOUT>), dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                     static_cast<u32x4_t*>(out0), static_cast<u32x4_t*>(out1), static_cast<const u32x4_t*>(in0),
                     static_cast<const u32x4_t*>(in1), vecs);
}

}  // namespace

// outs[0..nout), ins[0..nin): device pointers, 16-byte aligned, `vecs` 16-byte
// vectors each.  Returns 0 on success, 2 for bad counts or sizes, 1 for a NULL
// or misaligned pointer, 6 for a launch error.
extern "C" int synth_stream_copy(void* const* outs, int nout, const void* const* ins, int nin, int64_t vecs,
                                 hipStream_t stream) {
  if (nout < 1 || nout > 2 || nin < 1 || nin > 2 || vecs < 0 || vecs > (int64_t)0x7fffffff * kBlock) return 2;
  if (vecs == 0) return 0;
  if (outs == nullptr || ins == nullptr) return 1;
  for (int k = 0; k < nout; ++k)
    if (outs[k] == nullptr || (reinterpret_cast<uintptr_t>(outs[k]) & 15u)) return 1;
  for (int k = 0; k < nin; ++k)
    if (ins[k] == nullptr || (reinterpret_cast<uintptr_t>(ins[k]) & 15u)) return 1;
  void* o1 = nout == 2 ? outs[1] : nullptr;
  const void* i1 = nin == 2 ? ins[1] : nullptr;
  if (nin == 1 && nout == 1) launch<1, 1>(outs[0], o1, ins[0], i1, vecs, stream);
  if (nin == 2 && nout == 1) launch<2, 1>(outs[0], o1, ins[0], i1, vecs, stream);
  if (nin == 1 && nout == 2) launch<1, 2>(outs[0], o1, ins[0], i1, vecs, stream);
  if (nin == 2 && nout == 2) launch<2, 2>(outs[0], o1, ins[0], i1, vecs, stream);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
