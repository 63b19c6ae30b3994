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

// A lane's running state: its share (keys of its lane half) of the output
// accumulators and of the softmax denominator, and the row's running max.
template <int D>
struct AttnState {
  f32x16_t oacc[D / 32];
  float m;  // running max of the row's logits, base 2, shared by lanes l and l^32
  float l;  // sum of this lane's weights (FP32, unrounded), scaled to m
};

// Headroom, in base-2 units, the running max may lag the true max by: the
// output is rescaled only when a block raises the row max by more than this,
// so weights stay below 2^8 and the accumulators in FP32 range.
constexpr float kAttnLazyMax = 8.0f;

// One key block for one wave.  The scores come out of the MFMAs as
//   S = q.k + (key - k0) * slope/scale
// (the ALiBi offset inside the block enters as one more MFMA k-step, from the
// constant fragments kx and qx), so the base-2 logit is
//   t = S*scale2 + slope2*(k0 - q),
// the second term being one number per lane per block.  DIAG: some key of
// the block is after some query of the wave, so the causal mask applies.
template <int D, bool DIAG>
__device__ __forceinline__ void attn_block(AttnState<D>& st, const uint16_t* __restrict__ ksb,
                                           const uint16_t* __restrict__ vtb, const bf16x8_t (&qf)[D / 16],
                                           const bf16x8_t (&kx)[2], const bf16x8_t& qx, float scale2,
                                           float slope2, int k0, int qi, int half, int col) {
  constexpr int KS = D / 16, DT = D / 32, KROW = D + 8, VROW = kAttnBlockN + 8;
  // S^T tiles: keys k0 + 32*kt + (8*(i/4) + 4*half + i%4), query col.  The two
  // tiles' accumulation chains alternate, and the K fragments of step kk+1
  // are read while step kk's products run.
  const f32x16_t zero = {};
  f32x16_t s[2];
  s[0] = mfma32(kx[0], qx, zero);
  s[1] = mfma32(kx[1], qx, zero);
  const uint16_t* krow0 = &ksb[col * KROW + 8 * half];
  const uint16_t* krow1 = krow0 + 32 * KROW;
  uint4 a0 = *reinterpret_cast<const uint4*>(krow0);
  uint4 a1 = *reinterpret_cast<const uint4*>(krow1);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    uint4 n0 = a0, n1 = a1;
    if (kk + 1 < KS) {
      n0 = *reinterpret_cast<const uint4*>(krow0 + 16 * (kk + 1));
      n1 = *reinterpret_cast<const uint4*>(krow1 + 16 * (kk + 1));
    }
    s[0] = mfma32(as_bf16x8(a0), qf[kk], s[0]);
    s[1] = mfma32(as_bf16x8(a1), qf[kk], s[1]);
    a0 = n0;
    a1 = n1;
  }
  if (DIAG) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (k0 + 32 * kt + 8 * (i / 4) + 4 * half + (i % 4) > qi) s[kt][i] = -INFINITY;
  }
  // Row max: scale2 > 0, so the max of S*scale2 is scale2 times the max of S.
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
  const float shift = slope2 * (float)(k0 - qi);
  float bm = fmaf(mx, scale2, shift);
  bm = fmaxf(bm, __shfl_xor(bm, 32, kWave));
  if (__ballot(bm > st.m + kAttnLazyMax) != 0) {  // wave-uniform: rescale to a new max
    const float m_new = fmaxf(st.m, bm);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 on the first block
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.oacc[dt][i] *= alpha;
    st.l *= alpha;
    st.m = m_new;
  }
  const float c = fmaf(slope2, (float)(k0 - qi), -st.m);
  bf16x8_t pf[4];
  float l = st.l;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][i], scale2, c));
      l += p;
      pf[2 * kt + i / 8][i % 8] = (__bf16)p;
    }
  st.l = l;
  // O^T += V^T P^T over the 4 key steps of the block; the k order of step st
  // is keys 16*st + 4*half + {0..3, 8..11} for lane half `half` (key step
  // outer, head-dim tile inner: the DT accumulation chains alternate).
#pragma unroll
  for (int stp = 0; stp < 4; ++stp) {
    uint4 vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* row = &vtb[(dt * 32 + col) * VROW + 16 * stp + 4 * half];
      const uint2 lo = *reinterpret_cast<const uint2*>(row);
      const uint2 hi = *reinterpret_cast<const uint2*>(row + 8);
      vf[dt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.oacc[dt] = mfma32(as_bf16x8(vf[dt]), pf[stp], st.oacc[dt]);
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
  const bool wave_live = q0 < seq;

  // Q^T operand fragments: lane supplies q[qi][16*kk + 8*half .. +8].
  bf16x8_t qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const uint4 u = qvalid ? q[(base + qi) * VPR + 2 * kk + half] : make_uint4(0u, 0u, 0u, 0u);
    qf[kk] = as_bf16x8(u);
  }
  // ALiBi offset fragments: k-slots 0..2 of the lower lane half carry the key
  // offset in the block (an integer < 64, exact in bf16) against slope/scale
  // split into three bf16 parts; every other slot is zero.
  bf16x8_t kx[2], qx;
  {
    const float cs = slope2 / scale2;  // slope/scale
    const __bf16 c1 = (__bf16)cs;
    const float r1 = cs - (float)c1;
    const __bf16 c2 = (__bf16)r1;
    const __bf16 c3 = (__bf16)(r1 - (float)c2);
    const __bf16 z = (__bf16)0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool on = half == 0 && j < 3;
      qx[j] = on ? (j == 0 ? c1 : (j == 1 ? c2 : c3)) : z;
      kx[0][j] = on ? (__bf16)(float)col : z;
      kx[1][j] = on ? (__bf16)(float)(col + 32) : z;
    }
  }

  AttnState<D> st;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.oacc[dt][i] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;

  // Key blocks run from the diagonal back to key 0: the block holding a
  // row's own key comes first, and with the ALiBi bias falling off with
  // distance the running max then rarely moves.
  const int wg_last_q = min(seq, (qb + 1) * kAttnBlockM) - 1;
  const int nkb = wg_last_q / kAttnBlockN + 1;
  AttnStage<D> stage;
  attn_load<D>(stage, k, v, base, (nkb - 1) * kAttnBlockN, seq, t);
  attn_store<D>(stage, ks[0], vt[0], t);
  __syncthreads();
  for (int kb = nkb - 1, buf = 0; kb >= 0; --kb, buf ^= 1) {
    const int k0 = kb * kAttnBlockN;
    // next block's loads are in flight during this block's products
    if (kb > 0) attn_load<D>(stage, k, v, base, k0 - kAttnBlockN, seq, t);
    // Every processed block has k0 <= q0 (both are multiples of 32), so each
    // row has its key k0 unmasked and the first block sets a finite max.
    if (wave_live && k0 <= q0 + 31) {
      if (k0 + kAttnBlockN - 1 > q0)
        attn_block<D, true>(st, ks[buf], vt[buf], qf, kx, qx, scale2, slope2, k0, qi, half, col);
      else
        attn_block<D, false>(st, ks[buf], vt[buf], qf, kx, qx, scale2, slope2, k0, qi, half, col);
    }
    if (kb > 0) attn_store<D>(stage, ks[buf ^ 1], vt[buf ^ 1], t);
    __syncthreads();
  }

  // Normalise: the two lane halves hold the sums over complementary keys.
  const float l_tot = st.l + __shfl_xor(st.l, 32, kWave);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // d = 32*dt + 8*g + 4*half + 0..3
        const uint32_t lo = pack2(st.oacc[dt][4 * g] * inv, st.oacc[dt][4 * g + 1] * inv);
        const uint32_t hi = pack2(st.oacc[dt][4 * g + 2] * inv, st.oacc[dt][4 * g + 3] * inv);
        o[(base + qi) * (D / 4) + (32 * dt + 8 * g + 4 * half) / 4] = make_uint2(lo, hi);
      }
    }
    if (half == 0) lse[base + qi] = (st.m + __log2f(l_tot)) * 0.69314718055994530942f;
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
  BLOOM_REQUIRE(std::isfinite(scale) && scale >= 1e-30f, BLOOM_ERR_HPARAM, "scale = %g must be finite and >= 1e-30",
                (double)scale);
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
