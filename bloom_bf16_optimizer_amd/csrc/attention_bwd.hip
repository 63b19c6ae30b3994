// Fused causal attention with the ALiBi bias, backward, for gfx950.
//
// What is computed: the gradient of the attention of BLOOM's blocks (ALiBi
// bias of page "BLOOM 176B 训练技术概览", section "架构微调"; the combined
// scale + mask + softmax of "融合 CUDA 核" between Q K^T and V, run backward
// in training) for an upstream gradient dO, from q, k, v and the forward's
// log-sum-exp lse, without the L x L matrices:
//   p_ij  = exp(scale*(q_i . k_j) - slope_h*(i - j) - lse_i)   (j <= i, else 0)
//   dp_ij = dO_i . v_j,   D_i = sum_j p_ij dp_ij,   ds_ij = p_ij (dp_ij - D_i)
//   dq_i  = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
//   dv_j  = sum_i p_ij dO_i.
//
// Two kernels, each owning its outputs (no atomics, results independent of
// scheduling):
//  * query side (D and dq): a workgroup of four waves takes 128 consecutive
//    queries of one (b, h), a wave 32 (or, in launches with few query
//    blocks, 64 queries, a wave 32 of them against half the keys), and
//    streams the key blocks (64 keys, K and V staged in LDS) up to its
//    diagonal twice.  Both passes form S^T = K Q^T and dP^T = V dO^T so that
//    lane l owns query l%32 (its lse and D_i are one number each); as in the
//    forward, the ALiBi offset of a key within its 32-key half enters S^T as
//    one more MFMA k-step, so a score costs one FMA before exp2.  The first
//    sums D_i = sum_j p_ij dp_ij in FP32 and writes it to the workspace for
//    the dk/dv kernel; the second forms dS with that D and dQ^T += K^T dS^T
//    with K^T read from the same LDS tile by the transposing
//    ds_read_b64_tr_b16.  Each pass takes a block's 32-key halves one at a
//    time, so the kernel fits the 256 registers that let two waves share a
//    SIMD.
//    (The usual shortcut D_i = dO_i . o_i from the stored bf16 o carries that
//    rounding, 2^-9 of sum_d |dO_id o_id|, into every ds_ij of the row at
//    weight p_ij; with ALiBi's steep slopes p is often near 1 on the diagonal
//    and the error reaches the outputs.)
//  * dk/dv: a workgroup of eight waves takes 128 consecutive keys, two waves
//    per 32 keys, and streams the query blocks (64 queries, Q and dO staged in
//    LDS, with their lse and D) from its diagonal to the end.  One wave of a
//    pair forms S = Q K^T, P and dV^T += dO^T P; the other forms dP = dO V^T,
//    takes P through LDS, and forms dS and dK^T += Q^T dS, with dO^T and Q^T
//    read transposed from the staged tiles.  Lane l owns key l%32.
// Products use v_mfma_f32_32x32x16_bf16 with FP32 accumulation.  P enters
// as bf16 (it is >= 0, so its rounding stays relative to the result).  dS
// enters dQ and dK as two bf16 parts, hi = bf16(ds) and lo = bf16(ds - hi),
// i.e. with about 16 significant bits: dq and dk are sums of terms of both
// signs that can cancel to far below their size, where a single bf16
// rounding of ds (2^-9 of each term) would show in the result.  The
// exponentials are base 2 (scale, slopes and lse pre-multiplied by log2 e).
#include <cmath>
#include <type_traits>

#include "attention_common.h"

namespace bloom {
namespace {

constexpr int kBwdThreads = 256;  // four waves
constexpr int kBwdRows = 64;      // rows of a staged tile (keys for dq, queries for dk/dv)
constexpr int kBwdBlock = 128;    // keys per dk/dv item; queries per query-side item (or 64, see the launcher)
constexpr float kLog2e = 1.4426950408889634f;

// One staged tile: 64 rows of D bf16, row-major, written straight from global
// memory by global_load_lds_dwordx4.  Chunk c (16 bytes) of row r sits at
// c ^ swz(r).  The tiles are read two ways: one chunk per lane down 16
// consecutive rows (an MFMA operand with the row index on the lanes), and by
// the transposing read, two adjacent chunks (an even one and the next) of 4
// consecutive rows per 16-lane group.  swz keeps both free of bank conflicts:
// it takes 16 distinct values over 16 consecutive row groups (RPB rows share
// 256 bytes), and within 4 consecutive rows its values differ above bit 0.
template <int D>
struct BwdTile {
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
  static constexpr int RPB = 16 / CPR; // rows per 256 bytes
  static constexpr int Q4 = CPR / 4;
  static constexpr int CHUNKS = kBwdRows * CPR;
  __device__ static int swz(int r) {
    const int x = r / RPB;
    return 4 * (x % Q4) + (x / Q4) % 4;
  }
};

// Requests rows [r0, r0+64) of a [seq, D] matrix (row index base + r) into
// `tile`, moved by the first DW of the workgroup's NW waves: wave w < DW moves
// chunks [64*(DW*x + w), +64) for each x.  Rows past the end re-read row
// seq-1 (every use of them is masked).
template <int D, int NW = 4>
__device__ __forceinline__ void bwd_request(const uint4* __restrict__ g, attn_lds_uint4* tile, int64_t base, int r0,
                                           int seq, int w, int lane) {
  using T = BwdTile<D>;
  constexpr int DW = T::CHUNKS / kWave < NW ? T::CHUNKS / kWave : NW;
  constexpr int PER = T::CHUNKS / (DW * kWave);  // transfers per lane
  static_assert(PER >= 1 && T::CHUNKS % (DW * kWave) == 0, "tile size");
  if (w >= DW) return;  // wave-uniform
  const uint4* gb = attn_uniform(g + (base + r0) * T::CPR);
  const bool tail = r0 + kBwdRows > seq;  // wave-uniform
  if (!tail) {
    // Transfer x moves chunks DW*64*x further on in both the tile and the
    // rows: DW*64/CPR rows, a multiple of swz's period of 16 rows, so every
    // transfer has the first one's lane offset and a uniform step of DW KB.
    const int slot = w * kWave + lane;
    const int r = slot / T::CPR, c = (slot % T::CPR) ^ T::swz(r);
    const uint32_t vo = (uint32_t)(r * T::CPR + c) * 16u;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tile + w * kWave));
#pragma unroll
    for (int x = 0; x < PER; ++x) attn_dma16(gb + x * DW * kWave, vo, m0 + (uint32_t)(x * DW * kWave * 16));
    return;
  }
#pragma unroll
  for (int x = 0; x < PER; ++x) {
    const int first = (DW * x + w) * kWave;
    const int slot = first + lane;
    const int r = slot / T::CPR, pc = slot % T::CPR;
    const int c = pc ^ T::swz(r);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tile + first));
    const int row = min(r, seq - 1 - r0);
    attn_dma16(gb, (uint32_t)(row * T::CPR + c) * 16u, m0);
  }
}

// The A operand of an MFMA from a staged tile read transposed: lane L gets
// column d = 32*dt + L%32 of rows row0 + 4*(L/32) + {0..3} and of the same
// rows + 8, which is the k order of the P / dS fragments below.
template <int D>
__device__ __forceinline__ bf16x8_t bwd_read_tr(const char __attribute__((address_space(3)))* bytes, int row0, int dt,
                                                int trow, int tg, int tc, int sw0, int sw8) {
  const int cc = 4 * dt + 2 * tg + (tc >> 1);
  const int off0 = (row0 + trow) * (2 * D) + 16 * (cc ^ sw0) + 8 * (tc & 1);
  const int off8 = (row0 + trow + 8) * (2 * D) + 16 * (cc ^ sw8) + 8 * (tc & 1);
  const attn_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((attn_lds_v4s*)(bytes + off0));
  const attn_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((attn_lds_v4s*)(bytes + off8));
  const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
  return as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
}

// Two products a0*b0, a1*b1 as hi + lo pairs of bf16, packed two to a
// dword (element 0 in the low half): hi = RNE(a*b), lo = RNE(a*b - hi) with
// the residual formed by one fma from the exact product.
struct Bf16Split2 {
  uint32_t hi, lo;
};
__device__ __forceinline__ Bf16Split2 split_bf16x2(float a0, float b0, float a1, float b1) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t x = {a0 * b0, a1 * b1};
  const uint32_t hu = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
  const float h0 = __uint_as_float(hu << 16), h1 = __uint_as_float(hu & 0xffff0000u);
  const f32x2_t r = {fmaf(a0, b0, -h0), fmaf(a1, b1, -h1)};
  return {hu, __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t))};
}

// ---------------------------------------------------------------------------
// Query-side passes: one key block for one wave.  s, dp: rows = keys
// k0 + 32*kt + 8*(i/4) + 4*half + i%4, column = this lane's query qi.  The
// wave takes the block's 32-key halves kt0 .. kt0+NKT-1 (both, or one), one
// at a time, so that only one half's S, dP and dS are live.  SUM: the D pass,
// which only adds p * dp into dsum; otherwise the dq pass, which forms dS with
// the row's D = delta and accumulates dQ^T over the half's two 16-key steps
// right after forming it.
template <int D, bool DIAG, bool SUM, int NKT>
__device__ __forceinline__ void dq_block(f32x16_t (&acc)[D / 32], float& dsum,
                                         const attn_lds_uint4* __restrict__ kt_lds,
                                         const attn_lds_uint4* __restrict__ vt_lds, const bf16x8_t (&qf)[D / 16],
                                         const bf16x8_t (&df)[D / 16], const bf16x8_t& kx, const bf16x8_t& qx,
                                         float scale2, float slope2, float lse2,
                                         float delta, int k0, int kt0, int qi, int half, int col, int lane) {
  using T = BwdTile<D>;
  constexpr int KS = D / 16, DT = D / 32;
  const f32x16_t zero = {};
  const int sw = T::swz(col);  // also the swizzle of row col + 32
  const attn_lds_u32x4* k0r = reinterpret_cast<const attn_lds_u32x4*>(kt_lds) + col * T::CPR;
  const attn_lds_u32x4* v0r = reinterpret_cast<const attn_lds_u32x4*>(vt_lds) + col * T::CPR;
  // transposing reads of K for dQ^T += K^T dS^T
  const int tj = (lane & 15) >> 2, tc = lane & 3, tg = (lane >> 4) & 1;
  const int trow = 4 * half + tj;
  const int sw0 = T::swz(trow), sw8 = T::swz(trow + 8);  // the same for every step (rows + 16)
  const char __attribute__((address_space(3)))* kbytes =
      reinterpret_cast<const char __attribute__((address_space(3)))*>(kt_lds);
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int kt = kt0 + u;
    f32x16_t dp = zero;
    // the score products at a raised issue priority: the other wave of the
    // SIMD then fills the gaps of this chain instead of delaying it; the
    // first k-step adds the key's offset in the half times slope/scale
    __builtin_amdgcn_s_setprio(1);
    f32x16_t s = mfma32(kx, qx, zero);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int c = 32 * kt * T::CPR + ((2 * kk + half) ^ sw);
      s = mfma32(__builtin_bit_cast(bf16x8_t, k0r[c]), qf[kk], s);
      dp = mfma32(__builtin_bit_cast(bf16x8_t, v0r[c]), df[kk], dp);
    }
    __builtin_amdgcn_s_setprio(0);
    attn_u32x4 dsh[2], dsl[2];  // the bf16x8 operands of each part, as dwords
    float pp[2];
    // base-2 logit minus lse: s*scale2 + slope2*(k0 + 32*kt - qi) - lse2
    const float cb = fmaf(slope2, (float)(k0 + 32 * kt - qi), -lse2);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int off = 32 * kt + 8 * (i / 4) + (i % 4);  // key - k0 - 4*half
      float p = __builtin_amdgcn_exp2f(fmaf(s[i], scale2, cb));
      if (DIAG && k0 + 4 * half + off > qi) p = 0.f;
      if (SUM) {
        dsum = fmaf(p, dp[i], dsum);
      } else {
        pp[i & 1] = p;
        if (i & 1) {
          const Bf16Split2 d2 = split_bf16x2(pp[0], dp[i - 1] - delta, pp[1], dp[i] - delta);
          dsh[i / 8][(i % 8) / 2] = d2.hi;
          dsl[i / 8][(i % 8) / 2] = d2.lo;
        }
      }
    }
    if (!SUM) {
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8_t kT = bwd_read_tr<D>(kbytes, 16 * (2 * kt + st2), dt, trow, tg, tc, sw0, sw8);
          acc[dt] = mfma32(kT, __builtin_bit_cast(bf16x8_t, dsh[st2]), acc[dt]);
          acc[dt] = mfma32(kT, __builtin_bit_cast(bf16x8_t, dsl[st2]), acc[dt]);
        }
    }
  }
}

// The query-side kernel: a workgroup of four waves takes items of QI
// consecutive queries of one (b, h) and streams the key blocks (64 keys, K
// and V staged in LDS) from its diagonal down to key 0 twice: the D pass
// sums D_i = sum_j p_ij dp_ij for its queries (and writes it to `delta_out`
// for the dk/dv kernel), then the dq pass forms dS with that D, still in
// registers, and accumulates dQ^T.
// QI = 128: wave w takes queries 32w .. +31 against all 64 keys of a block.
// QI = 64: wave w takes queries 32*(w%2) .. +31 against the block's keys
// 32*(w/2) .. +31; the two waves of a query tile exchange their D sums and
// add their dQ halves through LDS (twice the items, for launches with few
// of them).
//
// Persistent workgroups, two per compute unit: a workgroup takes items
// (numbered longest first: item j is query block qblocks-1-j/bh_count of
// (b, h) = j % bh_count) in a snake over the grid (round r: item r*G + g for
// even r, r*G + G-1-g for odd r), so heavy items pair with light ones.  While
// a pass's last key block is used, the next pass's (or the next item's)
// first block is already on its way, and the next item's rows are loaded
// before this item's result is stored.
template <int D, int QI>
__device__ __forceinline__ void bwd_query_pass(const uint4* __restrict__ q, const uint4* __restrict__ k,
                                               const uint4* __restrict__ v, const uint4* __restrict__ dout,
                                               const float* __restrict__ lse, float* __restrict__ delta_out,
                                               uint2* __restrict__ dq, int seq, int heads, int qblocks, int bh_count,
                                               float scale2, float scale, const AttnSlopes& slopes) {
  static_assert(QI == 64 || QI == 128, "items of 64 or 128 queries");
  constexpr int KS = D / 16, DT = D / 32, VPR = D / 8;
  constexpr int CH = BwdTile<D>::CHUNKS;
  constexpr int NKT = QI / 64;  // 32-key halves of a block per wave
  __shared__ __attribute__((aligned(16))) uint4 tiles[2][2][CH];  // [stage][K, V]

  const int t = threadIdx.x;
  const int w = t / kWave, lane = t & (kWave - 1), half = lane >> 5, col = lane & 31;
  const int qt = QI == 128 ? w : (w & 1);  // this wave's 32-query tile within the item
  const int kh = QI == 128 ? 0 : (w >> 1);  // its first 32-key half of each block
  attn_lds_uint4* lt = (attn_lds_uint4*)&tiles[0][0][0];
  auto tile = [&](int stage, int which) { return lt + (stage * 2 + which) * CH; };

  const int G = (int)gridDim.x, g = (int)blockIdx.x;
  const int n_items = qblocks * bh_count;
  auto item_j = [&](int r) { return r * G + ((r & 1) ? G - 1 - g : g); };
  auto nkb_of = [&](int qb_) { return (min(seq, (qb_ + 1) * QI) - 1) / kBwdRows + 1; };

  int j = item_j(0);
  if (j >= n_items) return;  // uniform over the workgroup
  // B operands: this lane's query row of q and dO (d = 16*kk + 8*half .. +8)
  bf16x8_t qf[KS], df[KS];
  bf16x8_t kx[2];  // kx[0]: the key offset in a 32-key half (kx[1] unused)
  attn_key_offsets(kx, half, col);
  float lse2;
  auto load_rows = [&](int jn) {
    const int qb_ = qblocks - 1 - jn / bh_count;
    const int64_t bh_ = jn % bh_count;
    const int qi_ = qb_ * QI + qt * 32 + col;
    const bool ok = qi_ < seq;
    // rows past seq read row seq-1 and are then zeroed (no branches)
    const int64_t row = bh_ * (int64_t)seq + min(qi_, seq - 1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int64_t idx = row * VPR + 2 * kk + half;
      const uint4 a = q[idx], b = dout[idx];
      qf[kk] = as_bf16x8(ok ? a : make_uint4(0u, 0u, 0u, 0u));
      df[kk] = as_bf16x8(ok ? b : make_uint4(0u, 0u, 0u, 0u));
    }
    const float l = lse[row];
    lse2 = ok ? l * kLog2e : 0.f;
  };
  auto request_block = [&](int jn, int kb_, int stage) {
    const int64_t base_ = (int64_t)(jn % bh_count) * seq;
    bwd_request<D>(k, tile(stage, 0), base_, kb_ * kBwdRows, seq, w, lane);
    bwd_request<D>(v, tile(stage, 1), base_, kb_ * kBwdRows, seq, w, lane);
  };
  load_rows(j);
  request_block(j, nkb_of(qblocks - 1 - j / bh_count) - 1, 0);
  int buf = 0;  // the stage holding the next block to use
  for (int r = 0;; ++r) {
    const int qb = qblocks - 1 - j / bh_count;
    const int64_t bh = j % bh_count;
    const int h = (int)(bh % heads);
    const float slope2 = slopes.s[h];
    const bf16x8_t qx = attn_slope_parts(slope2, scale2, half);
    const int64_t base = bh * (int64_t)seq;
    const int q0 = qb * QI + qt * 32;  // this wave's first query
    const int qi = q0 + col;
    const bool qvalid = qi < seq;
    const bool wave_live = q0 < seq;
    const int jn = item_j(r + 1);
    const bool has_next = jn < n_items;
    const int nkb = nkb_of(qb);  // key blocks nkb-1 .. 0
    const bool writer = qvalid && kh == 0;

    // One pass over the item's key blocks (SUM: the D pass); during its last
    // block, block nkb_next-1 of item nj (if nvalid) is requested.
    auto walk = [&](auto sum_tag, f32x16_t(&acc)[DT], float& dsum, float delta, int nj, int nkb_next, bool nvalid) {
      constexpr bool SUM = decltype(sum_tag)::value;
      attn_wait_loads();
      __syncthreads();
      for (int kb = nkb - 1; kb >= 0; --kb, buf ^= 1) {
        const int k0 = kb * kBwdRows;
        const int kw0 = k0 + 32 * kh;  // this wave's first key of the block
        // the next block arrives while this one is used (the barrier that
        // ended the previous iteration freed its buffer)
        if (kb >= 1)
          request_block(j, kb - 1, buf ^ 1);
        else if (nvalid)
          request_block(nj, nkb_next - 1, buf ^ 1);
        if (wave_live && kw0 <= q0 + 31) {
          if (kw0 + 32 * NKT - 1 > q0)
            dq_block<D, true, SUM, NKT>(acc, dsum, tile(buf, 0), tile(buf, 1), qf, df, kx[0], qx, scale2, slope2,
                                        lse2, delta, k0, kh, qi, half, col, lane);
          else
            dq_block<D, false, SUM, NKT>(acc, dsum, tile(buf, 0), tile(buf, 1), qf, df, kx[0], qx, scale2, slope2,
                                         lse2, delta, k0, kh, qi, half, col, lane);
        }
        attn_wait_loads();
        __syncthreads();
      }
    };

    f32x16_t acc[DT];
    // the D pass; then the same item's first block is on its way again
    float dsum = 0.f;
    walk(std::integral_constant<bool, true>(), acc, dsum, 0.f, j, nkb, true);
    // the two lane halves summed complementary keys of the same query
    float dl = dsum + __shfl_xor(dsum, 32, kWave);
    if (QI == 64) {
      // both key-half waves of a query tile need the whole D: each hands its
      // sum to the other through the stage the last block used (added in the
      // same order on both sides)
      float* xch = reinterpret_cast<float*>(&tiles[buf ^ 1][0][0]) + qt * (2 * kWave);
      xch[kh * kWave + lane] = dl;
      __syncthreads();
      const float other = xch[(kh ^ 1) * kWave + lane];
      dl = kh == 0 ? dl + other : other + dl;
    }
    if (writer && half == 0) delta_out[base + qi] = dl;

    // the dq pass
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
    walk(std::integral_constant<bool, false>(), acc, dsum, qvalid ? dl : 0.f, jn,
         has_next ? nkb_of(qblocks - 1 - jn / bh_count) : 1, has_next);
    // The stage the last block used takes the dq rows (32-row groups QP
    // bytes apart) for stores of whole rows; with 64-query items the
    // key-half-1 waves first hand their dQ^T to the key-half-0 waves of the
    // same queries through the same memory, each tile's rows inside its own
    // hand-over area.
    constexpr int QP = QI == 64 ? DT * 16 * kWave * 4 : 32 * 2 * D;
    static_assert(QP >= 32 * 2 * D && (QI / 32) * QP <= 2 * CH * 16, "dq rows in one stage");
    char* stage_bytes = reinterpret_cast<char*>(&tiles[buf ^ 1][0][0]);
    if (QI == 64) {
      float* xch = reinterpret_cast<float*>(stage_bytes + qt * QP);
      if (kh == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) xch[(dt * 16 + i) * kWave + lane] = acc[dt][i];
      }
      __syncthreads();
      if (kh == 0) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dt][i] += xch[(dt * 16 + i) * kWave + lane];
      }
    }
    if (kh == 0) attn_stage_row<D>(acc, scale, stage_bytes, QP, qt * 32 + col, half);
    __syncthreads();
    attn_store_staged<D, QI, kBwdThreads>(stage_bytes, QP, dq, base + qb * QI, seq - qb * QI, t);
    // this item's q, dO and lse are no longer needed: the next item's load now
    if (has_next) load_rows(jn);
    if (!has_next) break;  // uniform over the workgroup
    j = jn;
  }
}

// D_i for every query (FP32, [b*h*seq], to `delta`) and
// dq_i = scale * sum_j ds_ij k_j.
template <int D, int QI>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void attention_bwd_query_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    const uint4* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ delta,
    uint2* __restrict__ dq, int seq, int heads, int qblocks, int bh_count, float scale2, float scale,
    AttnSlopes slopes) {
  bwd_query_pass<D, QI>(q, k, v, dout, lse, delta, dq, seq, heads, qblocks, bh_count, scale2, scale, slopes);
}

// ---------------------------------------------------------------------------
// dk/dv kernel.  A workgroup of eight waves takes 128 consecutive keys of one
// (b, h): waves w and w+4 own keys 32*(w%4) .. +31.  Wave w (the P wave) forms
// S = Q K^T and P for them and accumulates dV; wave w+4 (the dS wave) forms
// dP = dO V^T, takes P from the P wave through LDS, forms dS and accumulates
// dK.  Neither holds both accumulators, so two waves fit on a SIMD, and S is
// formed once.  Both stream the query blocks (64 queries, Q and dO staged in
// LDS with their lse and D) from the diagonal to the end, 32 queries (one
// tile) at a time, in two phases per block with a barrier between them:
//   phase 1: P waves S, P (stored to LDS) | dS waves dP
//   phase 2: P waves dV^T += dO^T P      | dS waves dS, dK^T += Q^T dS
// so that each SIMD runs one wave's products against the other's vector
// work; within a block the P waves run one 32-query tile ahead (three phases,
// see the walk below).  s, dp, p: rows = queries qt0 + 8*(i/4) + 4*half + i%4, column = this
// lane's key kj.  MASK: some key of the wave is after some query of the
// tile, or the tile runs past seq.

// P wave, phase 1: S = Q K^T and p = exp2(s*scale2 + bias - lse2) for one
// tile (rows tr0 .. tr0+31 of the staged 64, global queries qt0 ..); p goes
// to LDS as FP32 and into pf as bf16.
template <int D, bool MASK>
__device__ __forceinline__ void p_tile(bf16x8_t (&pf)[2], float4* __restrict__ pout,
                                       const attn_lds_uint4* __restrict__ q_lds,
                                       const float4* lse_lds, const bf16x8_t (&kf)[D / 16], float scale2, float slope2,
                                       int kj, int tr0, int qt0, int seq, int half, int col, int lane) {
  using T = BwdTile<D>;
  constexpr int KS = D / 16;
  f32x16_t s = {};
  const int sw = T::swz(tr0 + col);
  const attn_lds_u32x4* qr = reinterpret_cast<const attn_lds_u32x4*>(q_lds) + (tr0 + col) * T::CPR;
  __builtin_amdgcn_s_setprio(1);  // as in dq_block
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) s = mfma32(__builtin_bit_cast(bf16x8_t, qr[(2 * kk + half) ^ sw]), kf[kk], s);
  __builtin_amdgcn_s_setprio(0);
  // base-2 logit minus lse: s*scale2 + slope2*(kj - query) - lse2(query)
  const float cb = slope2 * (float)(kj - qt0 - 4 * half);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float4 l4 = lse_lds[(tr0 + 8 * g + 4 * half) / 4];
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
    float p4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;
      const int qoff = 8 * g + r;  // query - qt0 - 4*half
      float p = __builtin_amdgcn_exp2f(fmaf(s[i], scale2, fmaf(-slope2, (float)qoff, cb) - lv[r]));
      if (MASK) {
        const int qq = qt0 + 4 * half + qoff;
        if (kj > qq || qq >= seq) p = 0.f;
      }
      p4[r] = p;
      pf[i / 8][i % 8] = (__bf16)p;
    }
    pout[g * kWave + lane] = make_float4(p4[0], p4[1], p4[2], p4[3]);
  }
}

// P wave, phase 2: dV^T += dO^T P over the tile's 2 query steps.
template <int D>
__device__ __forceinline__ void dv_tile(f32x16_t (&dvacc)[D / 32], const bf16x8_t (&pf)[2],
                                        const attn_lds_uint4* __restrict__ do_lds, int tr0, int half, int lane) {
  using T = BwdTile<D>;
  constexpr int DT = D / 32;
  const int tj = (lane & 15) >> 2, tc = lane & 3, tg = (lane >> 4) & 1;
  const int trow = 4 * half + tj;
  const int sw0 = T::swz(trow), sw8 = T::swz(trow + 8);  // unchanged by row offsets that are multiples of 16
  const char __attribute__((address_space(3)))* dbytes =
      reinterpret_cast<const char __attribute__((address_space(3)))*>(do_lds);
#pragma unroll
  for (int stp = 0; stp < 2; ++stp)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      dvacc[dt] = mfma32(bwd_read_tr<D>(dbytes, tr0 + 16 * stp, dt, trow, tg, tc, sw0, sw8), pf[stp], dvacc[dt]);
}

// dS wave, phase 1: dP = dO V^T for one tile.
template <int D>
__device__ __forceinline__ f32x16_t dp_tile(const attn_lds_uint4* __restrict__ do_lds, const bf16x8_t (&vf)[D / 16],
                                            int tr0, int half, int col) {
  using T = BwdTile<D>;
  constexpr int KS = D / 16;
  f32x16_t dp = {};
  const int sw = T::swz(tr0 + col);
  const attn_lds_u32x4* dr = reinterpret_cast<const attn_lds_u32x4*>(do_lds) + (tr0 + col) * T::CPR;
  __builtin_amdgcn_s_setprio(1);  // as in dq_block
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) dp = mfma32(__builtin_bit_cast(bf16x8_t, dr[(2 * kk + half) ^ sw]), vf[kk], dp);
  __builtin_amdgcn_s_setprio(0);
  return dp;
}

// dS wave, phase 2: dS = P (dP - D) in two bf16 parts, dK^T += Q^T dS over
// the tile's 2 query steps.
template <int D>
__device__ __forceinline__ void dk_tile(f32x16_t (&dkacc)[D / 32], const f32x16_t& dp, const float4* __restrict__ pin,
                                        const attn_lds_uint4* __restrict__ q_lds, const float4* delta_lds, int tr0,
                                        int half, int lane) {
  using T = BwdTile<D>;
  constexpr int DT = D / 32;
  attn_u32x4 dsh[2], dsl[2];  // the bf16x8 operands of each part, as dwords
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float4 p4 = pin[g * kWave + lane];
    const float4 d4 = delta_lds[(tr0 + 8 * g + 4 * half) / 4];
    const float pv[4] = {p4.x, p4.y, p4.z, p4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      const int i = 4 * g + r;
      const Bf16Split2 d2 = split_bf16x2(pv[r], dp[i] - dv4[r], pv[r + 1], dp[i + 1] - dv4[r + 1]);
      dsh[i / 8][(i % 8) / 2] = d2.hi;
      dsl[i / 8][(i % 8) / 2] = d2.lo;
    }
  }
  const int tj = (lane & 15) >> 2, tc = lane & 3, tg = (lane >> 4) & 1;
  const int trow = 4 * half + tj;
  const int sw0 = T::swz(trow), sw8 = T::swz(trow + 8);
  const char __attribute__((address_space(3)))* qbytes =
      reinterpret_cast<const char __attribute__((address_space(3)))*>(q_lds);
#pragma unroll
  for (int stp = 0; stp < 2; ++stp)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bf16x8_t qT = bwd_read_tr<D>(qbytes, tr0 + 16 * stp, dt, trow, tg, tc, sw0, sw8);
      dkacc[dt] = mfma32(qT, __builtin_bit_cast(bf16x8_t, dsh[stp]), dkacc[dt]);
      dkacc[dt] = mfma32(qT, __builtin_bit_cast(bf16x8_t, dsl[stp]), dkacc[dt]);
    }
}

// An item of the dk/dv kernel (128 keys of one (b, h)), numbered heaviest
// first: hb is its key block (block 0 meets every query, so it is the
// heaviest), bh its (b, h).  With xs, item j belongs to XCD j % 8: every
// (b, h) is cut into its key blocks of either parity and XCD x takes
// half-heads [x*n, (x+1)*n), so an XCD's L2 holds the Q and dO of at most
// n/2 + 1 heads.  Otherwise items walk the key blocks from the first, every
// (b, h) at each step.
struct BwdItem {
  int hb;
  int64_t bh;
};
__device__ __forceinline__ BwdItem bwd_item(int j, int nblocks, int bh_count, bool xs) {
  BwdItem it;
  if (xs) {
    const int x = j % 8, jj = j / 8;
    const int n = bh_count / 4;  // half-heads per XCD
    const int rank = jj / n, hh = n * x + jj % n, par = hh & 1;
    it.bh = hh >> 1;
    it.hb = ((nblocks - 1 - par) & 1) + 2 * rank;
  } else {
    it.hb = j / bh_count;
    it.bh = j % bh_count;
  }
  return it;
}
// Item of round r for workgroup g of G: a snake over the grid, or with xs
// over the G/8 workgroups of g's XCD (workgroup g runs on XCD g % 8).
__device__ __forceinline__ int bwd_round_item(int r, int g, int G, bool xs) {
  if (!xs) return r * G + ((r & 1) ? G - 1 - g : g);
  const int U = G / 8, u = g / 8;
  return (r * U + ((r & 1) ? U - 1 - u : u)) * 8 + g % 8;
}

constexpr int kKvWaves = 8;
constexpr int kKvThreads = kKvWaves * kWave;

template <int D>
struct KvShared {
  uint4 tiles[2][2][BwdTile<D>::CHUNKS];  // [stage][Q, dO]
  float4 rowv[2][2][kBwdRows / 4];        // [stage][lse2, D] of the 64 queries
  float4 pbuf[2][4][4 * kWave];           // [tile][key group]: P, 16 values per lane
};

// One role's walk over the workgroup's items (DSW: the dS waves).  The two
// roles run the same sequence of barriers; every other step differs, so the
// role is a template parameter and each role's registers are allocated alone.
//
// Persistent workgroups, one per compute unit: a workgroup takes items (128
// keys of one (b, h), numbered longest first, see bwd_item) in a snake over
// its XCD's workgroups (xs) or over the grid.  The next block (or the next
// item's first block) is in flight while a block is used.
template <int D, bool DSW>
__device__ __forceinline__ void dkdv_walk(KvShared<D>& sh, const uint4* __restrict__ q, const uint4* __restrict__ k,
                                          const uint4* __restrict__ v, const uint4* __restrict__ dout,
                                          const float* __restrict__ lse, const float* __restrict__ delta,
                                          uint2* __restrict__ out, int seq, int heads, int kblocks, int bh_count,
                                          bool xs, float scale2, float outscale, const AttnSlopes& slopes) {
  constexpr int KS = D / 16, DT = D / 32, VPR = D / 8;
  constexpr int CH = BwdTile<D>::CHUNKS;
  const int t = threadIdx.x;
  const int w = t / kWave, lane = t & (kWave - 1), half = lane >> 5, col = lane & 31;
  const int kgrp = w % 4;  // this wave's 32 keys within the item
  attn_lds_uint4* lt = (attn_lds_uint4*)&sh.tiles[0][0][0];
  auto tile = [&](int stage, int which) { return lt + (stage * 2 + which) * CH; };

  const int G = (int)gridDim.x, g = (int)blockIdx.x;
  const int n_items = kblocks * bh_count;
  auto item_j = [&](int r) { return bwd_round_item(r, g, G, xs); };
  auto kb_of = [&](int jn) { return bwd_item(jn, kblocks, bh_count, xs).hb; };
  auto bh_of = [&](int jn) { return bwd_item(jn, kblocks, bh_count, xs).bh; };
  const int nqb = (seq + kBwdRows - 1) / kBwdRows;

  int j = item_j(0);
  if (j >= n_items) return;  // uniform over the workgroup

  // B operand: this lane's key row of k (P waves) or v (dS waves),
  // d = 16*kk + 8*half .. +8; keys past seq read row seq-1 and are zeroed
  bf16x8_t kv[KS];
  auto load_keys = [&](int jn) {
    const int kj_ = kb_of(jn) * kBwdBlock + kgrp * 32 + col;
    const bool ok = kj_ < seq;
    const int64_t row = bh_of(jn) * seq + min(kj_, seq - 1);
    const uint4* src = DSW ? v : k;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 a = src[row * VPR + 2 * kk + half];
      kv[kk] = as_bf16x8(ok ? a : make_uint4(0u, 0u, 0u, 0u));
    }
  };
  // Row values of a query block: lanes 0..15 of wave 0 (a P wave) move 4 lse
  // values each, lanes 16..31 4 values of D (groups past seq re-read the last
  // group; seq is a multiple of 8, so a group of 4 is wholly inside or outside).
  auto row_load = [&](int64_t base_, int r0) {
    const int grp = r0 + 4 * (t & 15);
    const int64_t at = base_ + min(grp, seq - 4);
    return (t < 16) ? *reinterpret_cast<const float4*>(lse + at) : *reinterpret_cast<const float4*>(delta + at);
  };
  auto row_store = [&](int stage, float4 x) {
    if (t < 16) x = make_float4(x.x * kLog2e, x.y * kLog2e, x.z * kLog2e, x.w * kLog2e);
    sh.rowv[stage][t >> 4][t & 15] = x;
  };
  auto request_block = [&](int64_t base_, int qb_, int stage) {
    bwd_request<D, kKvWaves>(q, tile(stage, 0), base_, qb_ * kBwdRows, seq, w, lane);
    bwd_request<D, kKvWaves>(dout, tile(stage, 1), base_, qb_ * kBwdRows, seq, w, lane);
  };
  auto first_qb = [&](int jn) { return (kb_of(jn) * kBwdBlock) / kBwdRows; };  // block of the item's first key

  load_keys(j);
  {
    const int64_t base0 = bh_of(j) * seq;
    request_block(base0, first_qb(j), 0);
    if (!DSW && t < 32) row_store(0, row_load(base0, first_qb(j) * kBwdRows));
  }
  int buf = 0;  // the stage holding the next block to use
  for (int r = 0;; ++r) {
    const int kb = kb_of(j);
    const int64_t bh = bh_of(j);
    const int h = (int)(bh % heads);
    const float slope2 = slopes.s[h];
    const int64_t base = bh * (int64_t)seq;
    const int kw0 = kb * kBwdBlock + kgrp * 32;  // this wave's first key
    const int kj = kw0 + col;
    const bool kvalid = kj < seq;
    const bool wave_live = kw0 < seq;
    const int jn = item_j(r + 1);
    const bool has_next = jn < n_items;

    f32x16_t acc[DT];  // dK^T (dS waves) or dV^T (P waves) of this wave's keys
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

    attn_wait_loads();
    __syncthreads();
    for (int qbi = first_qb(j); qbi < nqb; ++qbi, buf ^= 1) {
      const int q0 = qbi * kBwdRows;
      const bool next = qbi + 1 < nqb;
      // the next block (this item's, or the next item's first) arrives while
      // this one is used (the barrier that ended the previous iteration freed
      // its buffer)
      const bool rnext = next || has_next;
      const int64_t nbase = next || !has_next ? base : bh_of(jn) * seq;
      const int nqb0 = next ? qbi + 1 : (has_next ? first_qb(jn) : qbi);
      if (rnext) request_block(nbase, nqb0, buf ^ 1);
      // its row values (P waves, t < 32): one load, used only by the store at
      // the end of the block, so the compiler waits for it there and not
      // earlier (any earlier wait would also drain the transfers just issued)
      float4 rv;
      if (!DSW && t < 32) rv = row_load(nbase, nqb0 * kBwdRows);
      bool live[2], mask[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int qt0 = q0 + 32 * tt;
        live[tt] = wave_live && qt0 < seq && kw0 <= qt0 + 31;
        mask[tt] = kw0 + 31 > qt0 || qt0 + 32 > seq;
      }
      // three phases, one barrier between each: the P waves run one tile
      // ahead of the dS waves
      //   A: P waves S, P of tile 0           | dS waves dP of tiles 0 and 1
      //   B: P waves S, P of tile 1; dV tile 0 | dS waves dS, dK of tile 0
      //   C: P waves dV of tile 1             | dS waves dS, dK of tile 1
      if constexpr (DSW) {
        f32x16_t dpt[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          if (live[tt]) dpt[tt] = dp_tile<D>(tile(buf, 1), kv, 32 * tt, half, col);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          __syncthreads();  // the P waves' P of tile tt is in LDS
          if (live[tt]) dk_tile<D>(acc, dpt[tt], sh.pbuf[tt][kgrp], tile(buf, 0), sh.rowv[buf][1], 32 * tt, half, lane);
        }
      } else {
        bf16x8_t pf[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          if (live[tt]) {
            if (mask[tt])
              p_tile<D, true>(pf[tt], sh.pbuf[tt][kgrp], tile(buf, 0), sh.rowv[buf][0], kv, scale2, slope2, kj,
                              32 * tt, q0 + 32 * tt, seq, half, col, lane);
            else
              p_tile<D, false>(pf[tt], sh.pbuf[tt][kgrp], tile(buf, 0), sh.rowv[buf][0], kv, scale2, slope2, kj,
                               32 * tt, q0 + 32 * tt, seq, half, col, lane);
          }
          if (tt == 1 && live[0]) dv_tile<D>(acc, pf[0], tile(buf, 1), 0, half, lane);
          __syncthreads();  // P of tile tt is in LDS for the dS waves
        }
        if (live[1]) dv_tile<D>(acc, pf[1], tile(buf, 1), 32, half, lane);
        if (rnext && t < 32) row_store(buf ^ 1, rv);
      }
      attn_wait_loads();
      __syncthreads();
    }
    // dV rows through the stage the last block used, dK rows through the P
    // exchange, each stored as whole rows by the waves of its role
    char* rows = DSW ? reinterpret_cast<char*>(&sh.pbuf[0][0][0]) : reinterpret_cast<char*>(&sh.tiles[buf ^ 1][0][0]);
    static_assert(kBwdBlock * 2 * D <= sizeof(sh.pbuf) && kBwdBlock * 2 * D <= sizeof(sh.tiles[0]), "staged rows");
    attn_stage_row<D>(acc, outscale, rows, 32 * 2 * D, kgrp * 32 + col, half);
    __syncthreads();
    attn_store_staged<D, kBwdBlock, 4 * kWave>(rows, 32 * 2 * D, out, base + kb * kBwdBlock, seq - kb * kBwdBlock,
                                               t & (4 * kWave - 1));
    // this item's key rows are no longer needed: the next item's load now
    if (has_next) load_keys(jn);
    if (!has_next) break;  // uniform over the workgroup
    j = jn;
  }
}

template <int D>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2))) void attention_bwd_dkdv_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    const uint4* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    uint2* __restrict__ dk, uint2* __restrict__ dv, int seq, int heads, int kblocks, int bh_count, bool xs,
    float scale2, float scale, AttnSlopes slopes) {
  __shared__ __attribute__((aligned(16))) KvShared<D> sh;
  if (threadIdx.x >= 4 * kWave)  // wave-uniform: waves 4..7 are the dS waves
    dkdv_walk<D, true>(sh, q, k, v, dout, lse, delta, dk, seq, heads, kblocks, bh_count, xs, scale2, scale, slopes);
  else
    dkdv_walk<D, false>(sh, q, k, v, dout, lse, delta, dv, seq, heads, kblocks, bh_count, xs, scale2, 1.f, slopes);
}

size_t bwd_workspace(int64_t batch, int32_t heads, int64_t seq) {
  return ((size_t)(batch * heads * seq) * sizeof(float) + 255) / 256 * 256;
}

template <int D>
void launch_bwd(const bloom_bf16* q, const bloom_bf16* k, const bloom_bf16* v, const bloom_bf16* dout, const float* lse,
                bloom_bf16* dq, bloom_bf16* dk, bloom_bf16* dv,
                float* delta, int64_t batch, int32_t heads, int64_t seq, float scale2, float scale,
                const AttnSlopes& table, hipStream_t stream) {
  const int bh_count = (int)(batch * heads);
  const int blocks = (int)((seq + kBwdBlock - 1) / kBwdBlock);
  // the query-side kernel is persistent: two workgroups per compute unit, at
  // most one per item.  Items of 128 queries while they fill two rounds of
  // the grid, else of 64 (twice as many, so the causal work spreads evenly).
  const int64_t slots = 2 * (int64_t)(device_cu_count() > 0 ? device_cu_count() : 1);
  const bool wide = (int64_t)bh_count * blocks >= 2 * slots;
  const int qblocks = wide ? blocks : (int)((seq + 63) / 64);
  const int64_t n_items = (int64_t)bh_count * qblocks;
  const dim3 grid_q((unsigned)(n_items < slots ? n_items : slots));
  const uint4* qv = reinterpret_cast<const uint4*>(q);
  const uint4* kv = reinterpret_cast<const uint4*>(k);
  const uint4* vv = reinterpret_cast<const uint4*>(v);
  const uint4* dov = reinterpret_cast<const uint4*>(dout);
  if (wide)
    hipLaunchKernelGGL((attention_bwd_query_kernel<D, 128>), grid_q, dim3(kBwdThreads), 0, stream, qv, kv, vv, dov,
                       lse, delta, reinterpret_cast<uint2*>(dq), (int)seq, (int)heads, qblocks, bh_count, scale2,
                       scale, table);
  else
    hipLaunchKernelGGL((attention_bwd_query_kernel<D, 64>), grid_q, dim3(kBwdThreads), 0, stream, qv, kv, vv, dov,
                       lse, delta, reinterpret_cast<uint2*>(dq), (int)seq, (int)heads, qblocks, bh_count, scale2,
                       scale, table);
  // the dk/dv kernel is persistent too: one eight-wave workgroup per compute unit
  const int64_t kv_items = (int64_t)bh_count * blocks;
  const int64_t cus = slots / 2;
  // whole half-heads per XCD (an even number of key blocks, (b, h) pairs a
  // multiple of 4, a grid of whole XCD rounds): each XCD's L2 holds the Q
  // and dO of about a quarter of the heads it would otherwise stream
  const bool xs_kv = blocks % 2 == 0 && bh_count % 4 == 0 && cus % 8 == 0;
  const dim3 grid_kv((unsigned)(kv_items < cus ? kv_items : cus));
  hipLaunchKernelGGL((attention_bwd_dkdv_kernel<D>), grid_kv, dim3(kKvThreads), 0, stream, qv, kv, vv, dov, lse,
                     delta, reinterpret_cast<uint2*>(dk), reinterpret_cast<uint2*>(dv), (int)seq, (int)heads, blocks,
                     bh_count, xs_kv, scale2, scale, table);
}

}  // namespace
}  // namespace bloom

using namespace bloom;

extern "C" size_t bloom_alibi_attention_bwd_workspace_size(int64_t batch, int32_t heads, int64_t seq) {
  if (batch < 0 || heads < 0 || heads > BLOOM_MAX_HEADS || seq < 0 || seq > BLOOM_MAX_SEQ) return 0;
  if (batch * heads * seq == 0) return 256;
  return bwd_workspace(batch, heads, seq);
}

extern "C" bloom_status bloom_alibi_attention_bwd(const bloom_bf16* q, const bloom_bf16* k, const bloom_bf16* v,
                                                  const bloom_bf16* dout, const float* lse,
                                                  bloom_bf16* dq, bloom_bf16* dk, bloom_bf16* dv, int64_t batch,
                                                  int32_t heads, int64_t seq, int32_t head_dim,
                                                  int32_t head_offset, int32_t total_heads, float scale,
                                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  BLOOM_REQUIRE(batch >= 0 && heads >= 0, BLOOM_ERR_SHAPE, "batch and heads must be >= 0");
  BLOOM_REQUIRE(heads <= BLOOM_MAX_HEADS, BLOOM_ERR_SHAPE, "heads = %d exceeds %d", heads, BLOOM_MAX_HEADS);
  BLOOM_REQUIRE(seq >= 8 && seq <= BLOOM_MAX_SEQ && seq % 8 == 0, BLOOM_ERR_SHAPE,
                "seq = %lld must be a multiple of 8 in [8, %d]", (long long)seq, BLOOM_MAX_SEQ);
  BLOOM_REQUIRE(head_dim == 32 || head_dim == 64 || head_dim == 128, BLOOM_ERR_SHAPE,
                "head_dim = %d must be 32, 64 or 128", head_dim);
  BLOOM_REQUIRE(batch * heads * ((seq + kBwdBlock - 1) / kBwdBlock) <= 0x7fffffffLL, BLOOM_ERR_SHAPE,
                "too many blocks");
  BLOOM_REQUIRE(std::isfinite(scale) && scale >= 1e-30f, BLOOM_ERR_HPARAM, "scale = %g must be finite and >= 1e-30",
                (double)scale);
  BLOOM_REQUIRE(total_heads > 0 && head_offset >= 0 && (int64_t)head_offset + heads <= total_heads,
                BLOOM_ERR_SHAPE, "heads [%d, %d) outside a %d-head model", head_offset, head_offset + heads,
                total_heads);
  if (batch == 0 || heads == 0) return BLOOM_OK;
  BLOOM_REQUIRE_PTR(q);
  BLOOM_REQUIRE_PTR(k);
  BLOOM_REQUIRE_PTR(v);
  BLOOM_REQUIRE_PTR(dout);
  BLOOM_REQUIRE_PTR(lse);
  BLOOM_REQUIRE_PTR(dq);
  BLOOM_REQUIRE_PTR(dk);
  BLOOM_REQUIRE_PTR(dv);
  BLOOM_REQUIRE(workspace != nullptr, BLOOM_ERR_WORKSPACE, "workspace is NULL");
  BLOOM_REQUIRE(aligned16(workspace), BLOOM_ERR_ALIGN, "workspace is not 16-byte aligned");
  const size_t need = bwd_workspace(batch, heads, seq);
  BLOOM_REQUIRE(workspace_bytes >= need, BLOOM_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                need);
  float sl[BLOOM_MAX_HEADS];
  if (bloom_status st = bloom_alibi_slopes(total_heads, head_offset, heads, sl)) return st;
  AttnSlopes table;
  const double log2e = 1.4426950408889634;
  for (int hh = 0; hh < BLOOM_MAX_HEADS; ++hh) table.s[hh] = (hh < heads) ? (float)((double)sl[hh] * log2e) : 0.f;
  const float scale2 = (float)((double)scale * log2e);
  float* delta = static_cast<float*>(workspace);
  switch (head_dim) {
    case 32:
      launch_bwd<32>(q, k, v, dout, lse, dq, dk, dv, delta, batch, heads, seq, scale2, scale, table, stream);
      break;
    case 64:
      launch_bwd<64>(q, k, v, dout, lse, dq, dk, dv, delta, batch, heads, seq, scale2, scale, table, stream);
      break;
    default:
      launch_bwd<128>(q, k, v, dout, lse, dq, dk, dv, delta, batch, heads, seq, scale2, scale, table, stream);
      break;
  }
  return launch_status("bloom_alibi_attention_bwd");
}
