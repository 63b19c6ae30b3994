// Fused causal attention with the ALiBi bias (flash-style forward) for gfx950.
//
// What is computed: the attention of BLOOM's blocks with the ALiBi linear bias
// of page "BLOOM 176B 训练技术概览", section "架构微调" (trained at 2048
// tokens, extrapolated to 8192 in section 4.3 of page "企业官网建设流程全解析"),
// i.e. the combined scale + mask + softmax of "融合 CUDA 核" applied between
// Q K^T and V without materialising the L x L score tensor:
//   z_ij = scale*(q_i . k_j) - slope_h*(i - j) for j <= i (else masked),
//   o_i  = sum_j softmax_j(z_i) v_j,   lse_i = log sum_j exp(z_ij).
//
// Layout and mapping.  q, k, v, o are [B, NH, L, D] bf16 (D = 32, 64 or 128);
// a workgroup of four waves takes 128 consecutive queries of one (b, h), a
// wave 32 of them.  Keys are streamed in blocks of 64: K row-major and V
// transposed (V^T[d][key]) are staged in LDS, padded by 16 bytes per row.
// Matrix products use v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32, FP32
// accumulate; lane l supplies row/column l%32 and k-half l/32).  Scores are
// formed transposed, S^T = K Q^T, so that lane l owns query l%32: its scores
// for a 32-key tile sit in its 16 accumulator registers (keys
// 8*(i/4) + 4*(l/32) + i%4) and in those of lane l^32, so the online softmax
// is per lane plus one max exchange with lane l^32 per key block.  The
// output is formed transposed too, O^T += V^T P^T, with P^T taken straight
// from the score registers: the MFMA's k index runs over the 16 keys of a
// step in the order the registers hold them, and the V^T operand is read in
// that same order, so each lane also owns its query's 4*32 output values.
// The exponentials are base 2 (scale and slopes pre-multiplied by log2 e on
// the host); P is rounded to bf16 for the P V product.
#include <cmath>

#include "device_common.h"
#include "host_common.h"
#include "launch_plan.h"

namespace bloom {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kAttnBlockM = 128;  // queries per workgroup (4 waves x 32)
constexpr int kAttnBlockN = 64;   // keys per block
constexpr int kAttnThreads = 256;

struct AttnSlopes {
  float s[BLOOM_MAX_HEADS];  // slope_h * log2(e)
};

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// Per-thread share of one key block in flight: 16-byte vectors of K (row
// major) and of V (4 consecutive keys x 8 consecutive d, written to LDS
// transposed).
template <int D>
struct AttnStage {
  static constexpr int VPR = D / 8;                                  // 16-byte vectors per row
  static constexpr int KV = (kAttnBlockN * VPR) / kAttnThreads;      // K vectors per thread (>= 1)
  static constexpr int VGROUPS = (kAttnBlockN / 4) * VPR;            // (4-key group, d chunk) pairs
  uint4 kr[KV > 0 ? KV : 1];
  uint4 vr[4];
};

template <int D>
__device__ __forceinline__ void attn_load(AttnStage<D>& st, const uint4* __restrict__ k, const uint4* __restrict__ v,
                                          int64_t base, int k0, int seq, int t) {
  constexpr int VPR = AttnStage<D>::VPR;
#pragma unroll
  for (int r = 0; r < AttnStage<D>::KV; ++r) {
    const int idx = t + r * kAttnThreads;
    const int key = k0 + idx / VPR;
    st.kr[r] = key < seq ? k[(base + key) * VPR + idx % VPR] : make_uint4(0u, 0u, 0u, 0u);
  }
  if (t < AttnStage<D>::VGROUPS) {
    const int kg = t % (kAttnBlockN / 4), c = t / (kAttnBlockN / 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = k0 + 4 * kg + u;
      st.vr[u] = key < seq ? v[(base + key) * VPR + c] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

template <int D>
__device__ __forceinline__ void attn_store(const AttnStage<D>& st, uint16_t* ks, uint16_t* vt, int t) {
  constexpr int VPR = AttnStage<D>::VPR;
  constexpr int KROW = D + 8, VROW = kAttnBlockN + 8;
#pragma unroll
  for (int r = 0; r < AttnStage<D>::KV; ++r) {
    const int idx = t + r * kAttnThreads;
    *reinterpret_cast<uint4*>(&ks[(idx / VPR) * KROW + (idx % VPR) * 8]) = st.kr[r];
  }
  if (t < AttnStage<D>::VGROUPS) {
    const int kg = t % (kAttnBlockN / 4), c = t / (kAttnBlockN / 4);
    const uint32_t w0[4] = {st.vr[0].x, st.vr[0].y, st.vr[0].z, st.vr[0].w};
    const uint32_t w1[4] = {st.vr[1].x, st.vr[1].y, st.vr[1].z, st.vr[1].w};
    const uint32_t w2[4] = {st.vr[2].x, st.vr[2].y, st.vr[2].z, st.vr[2].w};
    const uint32_t w3[4] = {st.vr[3].x, st.vr[3].y, st.vr[3].z, st.vr[3].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // d = 8c + 2e takes the low halves of the four keys' words, d + 1 the high halves
      const uint2 lo = make_uint2(__builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u),
                                  __builtin_amdgcn_perm(w3[e], w2[e], 0x05040100u));
      const uint2 hi = make_uint2(__builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u),
                                  __builtin_amdgcn_perm(w3[e], w2[e], 0x07060302u));
      *reinterpret_cast<uint2*>(&vt[(8 * c + 2 * e) * VROW + 4 * kg]) = lo;
      *reinterpret_cast<uint2*>(&vt[(8 * c + 2 * e + 1) * VROW + 4 * kg]) = hi;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attention_fwd_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    uint2* __restrict__ o, float* __restrict__ lse, int seq, int heads, int qblocks, int bh_count,
    float scale2, AttnSlopes slopes) {
  constexpr int KS = D / 16;            // MFMA k-steps over the head dimension
  constexpr int DT = D / 32;            // 32-wide tiles of the head dimension
  constexpr int KROW = D + 8;           // padded K row (bf16)
  constexpr int VROW = kAttnBlockN + 8; // padded V^T row (bf16)
  constexpr int VPR = D / 8;            // 16-byte vectors per K/V row
  // two stages of K and V^T: the next key block is stored while this one is used
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kAttnBlockN * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][D * VROW];

  const int t = threadIdx.x;
  const int w = t / kWave, lane = t & (kWave - 1), half = lane >> 5, col = lane & 31;
  // Causal work grows with the query block: the grid walks query blocks from
  // the last (most keys) to the first, every (b, h) at each step, so the
  // longest workgroups are dispatched first and the short ones fill the tail.
  const int qb = qblocks - 1 - (int)(blockIdx.x / (unsigned)bh_count);
  const int64_t bh = blockIdx.x % (unsigned)bh_count;
  const int h = (int)(bh % heads);
  const float slope2 = slopes.s[h];
  const int64_t base = bh * (int64_t)seq;  // row index of (b, h, 0)
  const int q0 = qb * kAttnBlockM + w * 32;  // this wave's first query
  const int qi = q0 + col;                   // this lane's query
  const bool qvalid = qi < seq;

  // Q^T operand fragments: lane supplies q[qi][16*kk + 8*half .. +8].
  bf16x8_t qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const uint4 u = qvalid ? q[(base + qi) * VPR + 2 * kk + half] : make_uint4(0u, 0u, 0u, 0u);
    qf[kk] = as_bf16x8(u);
  }

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int wg_last_q = min(seq, (qb + 1) * kAttnBlockM) - 1;
  const int nkb = wg_last_q / kAttnBlockN + 1;
  AttnStage<D> stage;
  attn_load<D>(stage, k, v, base, 0, seq, t);
  attn_store<D>(stage, ks[0], vt[0], t);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * kAttnBlockN;
    const int buf = kb & 1;
    // next block's loads are in flight during this block's products
    if (kb + 1 < nkb) attn_load<D>(stage, k, v, base, k0 + kAttnBlockN, seq, t);

    if (k0 <= q0 + 31) {  // else every key of the block is after every query of this wave
      // S^T tiles: keys 32*kt + (8*(i/4) + 4*half + i%4), query col
      f32x16_t s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const uint4 a = *reinterpret_cast<const uint4*>(&ks[buf][(kt * 32 + col) * KROW + 16 * kk + 8 * half]);
          s[kt] = mfma32(as_bf16x8(a), qf[kk], s[kt]);
        }
      }
      // z = scale*s + slope*(j - qi), base 2; with j = k0 + 4*half + C_i and
      // C_i = 32*kt + 8*(i/4) + i%4 a constant, the bias is one fma per score.
      const float b0 = slope2 * (float)(k0 + 4 * half - qi);
      const bool diag = k0 + kAttnBlockN - 1 > q0;  // some key of the block is after some query
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ci = 32 * kt + 8 * (i / 4) + (i % 4);
          float z = fmaf(s[kt][i], scale2, fmaf(slope2, (float)ci, b0));
          if (diag && k0 + 4 * half + ci > qi) z = -INFINITY;
          s[kt][i] = z;
          mx = fmaxf(mx, z);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // a query past the end: all masked
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
      bf16x8_t pf[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[kt][i] - m_use);
          psum += p;
          pf[2 * kt + i / 8][i % 8] = (__bf16)p;
        }
      }
      l_run = fmaf(l_run, alpha, psum);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      // O^T += V^T P^T over the 4 key steps of the block; the k order of step
      // st is keys 16*st + 4*half + {0..3, 8..11} for lane half `half`.
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const uint16_t* row = &vt[buf][(dt * 32 + col) * VROW + 16 * st + 4 * half];
          const uint2 lo = *reinterpret_cast<const uint2*>(row);
          const uint2 hi = *reinterpret_cast<const uint2*>(row + 8);
          oacc[dt] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pf[st], oacc[dt]);
        }
      }
    }
    if (kb + 1 < nkb) attn_store<D>(stage, ks[buf ^ 1], vt[buf ^ 1], t);
    __syncthreads();
  }

  // Normalise: the two lane halves hold the sums over complementary keys.
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // d = 32*dt + 8*g + 4*half + 0..3
        const uint32_t lo = pack2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv);
        const uint32_t hi = pack2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
        o[(base + qi) * (D / 4) + (32 * dt + 8 * g + 4 * half) / 4] = make_uint2(lo, hi);
      }
    }
    if (half == 0) {
      const float m_fin = (m_run == -INFINITY) ? 0.f : m_run;
      lse[base + qi] = (m_fin + __log2f(l_tot)) * 0.69314718055994530942f;
    }
  }
}

bloom_status check_attention(int64_t batch, int32_t heads, int64_t seq, int32_t head_dim) {
  BLOOM_REQUIRE(batch >= 0 && heads >= 0, BLOOM_ERR_SHAPE, "batch and heads must be >= 0");
  BLOOM_REQUIRE(heads <= BLOOM_MAX_HEADS, BLOOM_ERR_SHAPE, "heads = %d exceeds %d", heads, BLOOM_MAX_HEADS);
  BLOOM_REQUIRE(seq >= 8 && seq <= BLOOM_MAX_SEQ && seq % 8 == 0, BLOOM_ERR_SHAPE,
                "seq = %lld must be a multiple of 8 in [8, %d]", (long long)seq, BLOOM_MAX_SEQ);
  BLOOM_REQUIRE(head_dim == 32 || head_dim == 64 || head_dim == 128, BLOOM_ERR_SHAPE,
                "head_dim = %d must be 32, 64 or 128", head_dim);
  const int64_t qblocks = (seq + kAttnBlockM - 1) / kAttnBlockM;
  BLOOM_REQUIRE(batch * heads * qblocks <= 0x7fffffffLL, BLOOM_ERR_SHAPE, "too many query blocks");
  return BLOOM_OK;
}

}  // namespace
}  // namespace bloom

using namespace bloom;

extern "C" bloom_status bloom_alibi_attention_fwd(const bloom_bf16* q, const bloom_bf16* k,
                                                  const bloom_bf16* v, bloom_bf16* o, float* lse,
                                                  int64_t batch, int32_t heads, int64_t seq,
                                                  int32_t head_dim, int32_t head_offset,
                                                  int32_t total_heads, float scale, hipStream_t stream) {
  clear_error();
  if (bloom_status st = check_attention(batch, heads, seq, head_dim)) return st;
  BLOOM_REQUIRE(std::isfinite(scale), BLOOM_ERR_HPARAM, "scale must be finite");
  BLOOM_REQUIRE(total_heads > 0 && head_offset >= 0 && (int64_t)head_offset + heads <= total_heads,
                BLOOM_ERR_SHAPE, "heads [%d, %d) outside a %d-head model", head_offset, head_offset + heads,
                total_heads);
  if (batch == 0 || heads == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(q);
  BLOOM_REQUIRE_PTR(k);
  BLOOM_REQUIRE_PTR(v);
  BLOOM_REQUIRE_PTR(o);
  BLOOM_REQUIRE_PTR(lse);
  float sl[BLOOM_MAX_HEADS];
  if (bloom_status st = bloom_alibi_slopes(total_heads, head_offset, heads, sl)) return st;
  AttnSlopes table;
  const double log2e = 1.4426950408889634;
  for (int hh = 0; hh < BLOOM_MAX_HEADS; ++hh) table.s[hh] = (hh < heads) ? (float)((double)sl[hh] * log2e) : 0.f;
  const float scale2 = (float)((double)scale * log2e);
  const int qblocks = (int)((seq + kAttnBlockM - 1) / kAttnBlockM);
  const dim3 grid((unsigned)(batch * heads * qblocks));
  const uint4* qv = reinterpret_cast<const uint4*>(q);
  const uint4* kv = reinterpret_cast<const uint4*>(k);
  const uint4* vv = reinterpret_cast<const uint4*>(v);
  uint2* ov = reinterpret_cast<uint2*>(o);
  switch (head_dim) {
    case 32:
      hipLaunchKernelGGL((attention_fwd_kernel<32>), grid, dim3(kAttnThreads), 0, stream, qv, kv, vv, ov, lse,
                         (int)seq, (int)heads, qblocks, (int)(batch * heads), scale2, table);
      break;
    case 64:
      hipLaunchKernelGGL((attention_fwd_kernel<64>), grid, dim3(kAttnThreads), 0, stream, qv, kv, vv, ov, lse,
                         (int)seq, (int)heads, qblocks, (int)(batch * heads), scale2, table);
      break;
    default:
      hipLaunchKernelGGL((attention_fwd_kernel<128>), grid, dim3(kAttnThreads), 0, stream, qv, kv, vv, ov, lse,
                         (int)seq, (int)heads, qblocks, (int)(batch * heads), scale2, table);
      break;
  }
  return launch_status("bloom_alibi_attention_fwd");
}
