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
// Layout and mapping.  q, k, v, o are [B, NH, L, D] bf16 (D = 32, 64 or 128).
// An item is 128 consecutive queries of one (b, h); a workgroup of eight
// waves (two key streams of four, a wave per 32 queries in each) works
// through a fixed list of items, one workgroup per compute unit, and starts
// the next item's Q and first key blocks while it merges and stores the
// current one.  Keys are streamed in blocks of 64 through unpadded,
// XOR-swizzled row-major K and V tiles in LDS (V read transposed).
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

#include "attention_common.h"
#include "launch_plan.h"

namespace bloom {
namespace {

constexpr int kAttnBlockM = 128;       // queries per workgroup (4 waves x 32)
constexpr int kAttnBlockN = 64;        // keys per block
constexpr int kAttnGroupThreads = 256; // one key stream: 4 waves, one per 32 queries
constexpr int kAttnThreads = 2 * kAttnGroupThreads;  // two key streams over the same queries

// One key block of K or V in LDS: 64 rows of D bf16, row-major, unpadded,
// written straight from global memory by global_load_lds_dwordx4 (each lane
// of a wave moves one 16-byte chunk to LDS address m0 + lane*16).  Within a
// row the 16-byte chunks are XOR-swizzled so that the two read patterns are
// free of bank conflicts:
//  - K is read one chunk per lane down 16 consecutive rows (the A operand of
//    the score MFMA): chunk c of row r sits at c ^ ((r / RPB) % CPR), so 16
//    rows spread over 16 different 4-bank groups;
//  - V is read with the transposing ds_read_b64_tr_b16, 64 bytes of each of
//    4 consecutive rows at a time: chunk c of row r sits at
//    c ^ 4*((r / RPB) % (CPR/4)), so those 4 rows occupy disjoint banks.
template <int D>
struct AttnTile {
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int RPB = 16 / CPR;                   // rows per 256 bytes
  static constexpr int CHUNKS = kAttnBlockN * CPR;       // chunks per tile
  static constexpr int DMA = CHUNKS / kAttnGroupThreads; // transfers per lane per tile
  static_assert(DMA >= 1 && CHUNKS % kAttnGroupThreads == 0, "tile / stream size");
  __device__ static int swz_k(int r) { return (r / RPB) % CPR; }
  __device__ static int swz_v(int r) { return 4 * ((r / RPB) % (CPR / 4)); }
};

// Requests key block [k0, k0+64) of K (SWZ_V false) or V into `tile`; this
// wave (wq of the stream's four) moves chunks [64*(4x + wq), +64) for each
// x.  A lane's chunk offset within the block does not depend on k0 or x (so
// it stays in a register across blocks); only the block at the end of the
// sequence re-reads row seq-1 for its rows past the end (their keys are
// masked for every query that is stored).
template <int D, bool SWZ_V>
__device__ __forceinline__ void attn_request(const uint4* __restrict__ g, attn_lds_uint4* tile, int64_t base, int k0,
                                             int seq, int wq, int lane) {
  using T = AttnTile<D>;
  const uint64_t gp = (uint64_t)(uintptr_t)(g + (base + k0) * T::CPR);
  const uint4* gb = (const uint4*)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(gp >> 32)) << 32) |
                                               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gp));
  const bool tail = k0 + kAttnBlockN > seq;  // wave-uniform
  if (!tail) {
    // Transfer x moves 256 chunks further on in both the block and its
    // rows: 256/CPR rows, a multiple of both swizzles' periods (16 and 4
    // rows), so every transfer has the first one's lane offset and a
    // uniform step of 4 KB in the scalar base and in m0.
    const int slot = wq * kWave + lane;
    const int r = slot / T::CPR, c = (slot % T::CPR) ^ (SWZ_V ? T::swz_v(r) : T::swz_k(r));
    const uint32_t vo = (uint32_t)(r * T::CPR + c) * 16u;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tile + wq * kWave));
#pragma unroll
    for (int x = 0; x < T::DMA; ++x)
      attn_dma16(gb + x * kAttnGroupThreads, vo, m0 + (uint32_t)(x * kAttnGroupThreads * 16));
    return;
  }
#pragma unroll
  for (int x = 0; x < T::DMA; ++x) {
    const int first = (4 * x + wq) * kWave;
    const int slot = first + lane;
    const int r = slot / T::CPR, pc = slot % T::CPR;
    const int c = pc ^ (SWZ_V ? T::swz_v(r) : T::swz_k(r));
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tile + first));
    const int row = min(r, seq - 1 - k0);
    attn_dma16(gb, (uint32_t)(row * T::CPR + c) * 16u, m0);
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
template <int D, bool DIAG, bool OPT = false>
__device__ __forceinline__ void attn_block(AttnState<D>& st, const attn_lds_uint4* __restrict__ kt_lds,
                                           const attn_lds_uint4* __restrict__ vt_lds, const bf16x8_t (&qf)[D / 16],
                                           const bf16x8_t (&kx)[2], const bf16x8_t& qx, float scale2,
                                           float slope2, int k0, int qi, int half, int col, int lane) {
  using T = AttnTile<D>;
  constexpr int KS = D / 16, DT = D / 32;
  // S^T tiles: keys k0 + 32*kt + (8*(i/4) + 4*half + i%4), query col.  Lane
  // reads chunk 2*kk + half of K rows col and 32 + col (same swizzle).
  const f32x16_t zero = {};
  f32x16_t s[2];
  // the score products at a raised issue priority: the other wave of the
  // SIMD then fills the gaps of this chain instead of delaying it
  __builtin_amdgcn_s_setprio(1);
  s[0] = mfma32(kx[0], qx, zero);
  s[1] = mfma32(kx[1], qx, zero);
  const int sk = T::swz_k(col);
  const attn_lds_u32x4* krow0 = reinterpret_cast<const attn_lds_u32x4*>(kt_lds) + col * T::CPR;
  const attn_lds_u32x4* krow1 = krow0 + 32 * T::CPR;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int c = (2 * kk + half) ^ sk;
    const attn_u32x4 a0 = krow0[c], a1 = krow1[c];
    s[0] = mfma32(__builtin_bit_cast(bf16x8_t, a0), qf[kk], s[0]);
    s[1] = mfma32(__builtin_bit_cast(bf16x8_t, a1), qf[kk], s[1]);
  }
  __builtin_amdgcn_s_setprio(0);
  if (DIAG) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (k0 + 32 * kt + 8 * (i / 4) + 4 * half + (i % 4) > qi) s[kt][i] = -INFINITY;
  }
  bf16x8_t pf[4];
  // The block's row max and a rescale when it exceeds the running max by
  // more than kAttnLazyMax (true if it rescaled).
  auto exact = [&]() {
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
      return true;
    }
    return false;
  };
  // The block's weights against the running max, into pf; returns the
  // running sum with them added.
  auto weights = [&]() {
    const float c = fmaf(slope2, (float)(k0 - qi), -st.m);
    float l = st.l;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][i], scale2, c));
        l += p;
        pf[2 * kt + i / 8][i % 8] = (__bf16)p;
      }
    return l;
  };
  float l;
  if (DIAG || !OPT) {
    exact();
    l = weights();
  } else {
    // OPT (callers whose waves reach every off-diagonal block after their
    // diagonal one, so the running max is set): away from the diagonal the
    // ALiBi bias keeps the logits below the running max, so the weights are
    // formed against it directly.  If a lane's block sum passes 2^7 (every
    // weight above 2^8 does), the block is redone the exact way; where that
    // way would not rescale, its weights are these ones.  Either way the
    // result is the exact way's.
    l = weights();
    if (__ballot(!(l - st.l <= 128.f)) != 0 && exact()) l = weights();
  }
  st.l = l;
  // O^T += V^T P^T over the 4 key steps of the block; the k order of step
  // stp is keys 16*stp + 4*half + {0..3, 8..11} for lane half `half`.  The
  // V^T operand comes from two transposing reads: lane L addresses 4
  // consecutive d (d0 = 32*dt + 16*((L/16)%2) + 4*(L%4)) of key row
  // 16*stp + 4*(L/32) + (L%16)/4 (+8 for the second read), and receives its
  // own d = 32*dt + L%32 for the four keys the lanes of its 16-group
  // addressed (key step outer, head-dim tile inner: the DT accumulation
  // chains alternate).
  const int tj = (lane & 15) >> 2, tc = lane & 3, tg = (lane >> 4) & 1;
  const int trow = 4 * half + tj;                 // + 16*stp (+ 8)
  const int tsv = T::swz_v(trow);                 // the same for every stp and the +8 row
  const char __attribute__((address_space(3)))* vbytes =
      reinterpret_cast<const char __attribute__((address_space(3)))*>(vt_lds);
#pragma unroll
  for (int stp = 0; stp < 4; ++stp) {
    bf16x8_t vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int cc = (4 * dt + 2 * tg + (tc >> 1)) ^ tsv;
      const int off = (16 * stp + trow) * (2 * D) + 16 * cc + 8 * (tc & 1);
      const attn_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((attn_lds_v4s*)(vbytes + off));
      const attn_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((attn_lds_v4s*)(vbytes + off + 8 * 2 * D));
      const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
      vf[dt] = as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.oacc[dt] = mfma32(vf[dt], pf[stp], st.oacc[dt]);
  }
}

// An item: 128 consecutive queries (query block qb) of one (b, h).  Items are
// numbered heaviest first (the causal work grows with the query block).  With
// xcd_split, item j belongs to XCD j % 8: every (b, h) is cut into its even
// and odd query blocks and XCD x takes half-heads [x*n, (x+1)*n), so an XCD's
// L2 holds the K and V of at most n/2 + 1 heads.  Otherwise items walk query
// blocks from the last to the first, every (b, h) at each step.
struct AttnItem {
  int qb;
  int64_t bh;
};
__device__ __forceinline__ AttnItem attn_item(int j, int qblocks, int bh_count, bool xcd_split) {
  AttnItem it;
  if (xcd_split) {
    const int x = j % 8, jj = j / 8;
    const int n = bh_count / 4;  // half-heads per XCD
    const int rank = jj / n, hh = n * x + jj % n, par = hh & 1;
    it.bh = hh >> 1;
    it.qb = qblocks - 1 - ((qblocks - 1 - par) & 1) - 2 * rank;
  } else {
    it.qb = qblocks - 1 - j / bh_count;
    it.bh = j % bh_count;
  }
  return it;
}

// Q^T operand fragments of a query row: lane supplies q[row][16*kk + 8*half .. +8]
// (zeros past the sequence).
template <int D>
__device__ __forceinline__ void attn_load_q(bf16x8_t (&qf)[D / 16], const uint4* __restrict__ q, int64_t row, bool ok,
                                            int half) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const uint4 u = ok ? q[row * (D / 8) + 2 * kk + half] : make_uint4(0u, 0u, 0u, 0u);
    qf[kk] = as_bf16x8(u);
  }
}

template <int D>
__device__ __forceinline__ void attn_state_init(AttnState<D>& st) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.oacc[dt][i] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;
}

// A finished row, normalised, into the staged output tile (attn_stage_row:
// the two lane halves hold the sums over complementary keys), and its lse
// (natural log) if ok.
template <int D>
__device__ __forceinline__ void attn_row_to_tile(const AttnState<D>& st, char* otile, int row, float* __restrict__ lse,
                                                 int64_t lrow, bool ok, int half) {
  const float l_tot = st.l + __shfl_xor(st.l, 32, kWave);
  attn_stage_row<D>(st.oacc, 1.0f / l_tot, otile, 32 * 2 * D, row, half);
  if (ok && half == 0) lse[lrow] = (st.m + __log2f(l_tot)) * 0.69314718055994530942f;
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void attention_fwd_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    uint2* __restrict__ o, float* __restrict__ lse, int seq, int heads, int qblocks, int bh_count,
    bool xcd_split, float scale2, AttnSlopes slopes) {
  constexpr int KS = D / 16;            // MFMA k-steps over the head dimension
  constexpr int DT = D / 32;            // 32-wide tiles of the head dimension
  constexpr int CH = AttnTile<D>::CHUNKS;
  // [stage][stream][K, V] tiles: the next pair of key blocks arrives while
  // this pair is used.  At the end of an item the same memory carries stream
  // 1's partial results to stream 0.
  __shared__ __attribute__((aligned(16))) uint4 tiles[2][2][2][CH];
  static_assert(sizeof(tiles) >= 4 * (DT * 16 + 2) * kWave * sizeof(float), "merge area");

  // Two streams of four waves take the same 128 queries (wave w and w+4 the
  // same 32) and alternate over the key blocks, so an item's serial chain is
  // half its key blocks; their partial softmax states merge at the end.
  const int t = threadIdx.x;
  const int w = t / kWave, lane = t & (kWave - 1), half = lane >> 5, col = lane & 31;
  const int stream = w >> 2, wq = w & 3;
  attn_lds_uint4* lt = (attn_lds_uint4*)&tiles[0][0][0][0];
  auto tile = [&](int stage, int which) { return lt + ((stage * 2 + stream) * 2 + which) * CH; };
  bf16x8_t kx[2];
  attn_key_offsets(kx, half, col);

  // Persistent workgroups: the grid is a multiple of 8 and workgroup g runs
  // on XCD g % 8.  The U workgroups of an XCD take its items (j % 8 == x) in
  // a snake (round r: local item r*U + u for even r, r*U + U-1-u for odd r),
  // which pairs heavy items with light ones.
  const int U = (int)(gridDim.x / 8u), x8 = (int)(blockIdx.x % 8u), u = (int)(blockIdx.x / 8u);
  const int n_items = qblocks * bh_count;
  auto item_index = [&](int r) { return (r * U + ((r & 1) ? U - 1 - u : u)) * 8 + x8; };
  auto nkb_of = [&](int qb_) { return (min(seq, (qb_ + 1) * kAttnBlockM) - 1) / kAttnBlockN + 1; };
  // The first key block of an item for this stream (none if the item has
  // fewer blocks than streams), into stage 0.
  auto request_first = [&](const AttnItem& it) {
    const int kb_ = nkb_of(it.qb) - 1 - stream;
    if (kb_ >= 0) {
      const int64_t base_ = it.bh * (int64_t)seq;
      attn_request<D, false>(k, tile(0, 0), base_, kb_ * kAttnBlockN, seq, wq, lane);
      attn_request<D, true>(v, tile(0, 1), base_, kb_ * kAttnBlockN, seq, wq, lane);
    }
  };
  auto q_row = [&](const AttnItem& it) { return it.qb * kAttnBlockM + wq * 32 + col; };

  int j = item_index(0);
  if (j >= n_items) return;  // uniform over the workgroup
  AttnItem cur = attn_item(j, qblocks, bh_count, xcd_split);
  bf16x8_t qf[KS];
  attn_load_q<D>(qf, q, cur.bh * (int64_t)seq + q_row(cur), q_row(cur) < seq, half);
  request_first(cur);
  for (int r = 0;; ++r) {
    const int qb = cur.qb;
    const int64_t base = cur.bh * (int64_t)seq;  // row index of (b, h, 0)
    const float slope2 = slopes.s[(int)(cur.bh % heads)];
    const int q0 = qb * kAttnBlockM + wq * 32;  // this wave's first query
    const int qi = q0 + col;                    // this lane's query
    const bool wave_live = q0 < seq;
    const bf16x8_t qx = attn_slope_parts(slope2, scale2, half);
    AttnState<D> st;
    attn_state_init(st);

    // Key blocks run from the diagonal back to key 0 (stream s takes blocks
    // nkb-1-s, nkb-3-s, ...): the block holding a row's own key comes first,
    // and with the ALiBi bias falling off with distance the running max then
    // rarely moves.  The first ones were requested already.
    const int nkb = nkb_of(qb);
    const int iters = (nkb + 1) / 2;
    int kb = nkb - 1 - stream;
    attn_wait_loads();
    __syncthreads();
    for (int it = 0, buf = 0; it < iters; ++it, buf ^= 1, kb -= 2) {
      const int k0 = kb * kAttnBlockN;
      // the next block's transfers run during this block's products (the
      // barrier that ended the previous iteration freed their buffer)
      if (kb >= 2) {
        attn_request<D, false>(k, tile(buf ^ 1, 0), base, k0 - 2 * kAttnBlockN, seq, wq, lane);
        attn_request<D, true>(v, tile(buf ^ 1, 1), base, k0 - 2 * kAttnBlockN, seq, wq, lane);
      }
      // Every processed block has k0 <= q0 (both are multiples of 32), so each
      // row has its key k0 unmasked and the first block sets a finite max.
      if (kb >= 0 && wave_live && k0 <= q0 + 31) {
        if (k0 + kAttnBlockN - 1 > q0)
          attn_block<D, true>(st, tile(buf, 0), tile(buf, 1), qf, kx, qx, scale2, slope2, k0, qi, half, col, lane);
        else
          attn_block<D, false>(st, tile(buf, 0), tile(buf, 1), qf, kx, qx, scale2, slope2, k0, qi, half, col, lane);
      }
      attn_wait_loads();
      __syncthreads();
    }

    const int jn = item_index(r + 1);
    const bool has_next = jn < n_items;
    const AttnItem nxt = attn_item(has_next ? jn : j, qblocks, bh_count, xcd_split);

    // Merge stream 1 into stream 0 through LDS ([wave][value][lane] floats).
    // Block 0 is processed by one of the streams for every live row, so at
    // least one of the two maxima is finite.
    float* mg = reinterpret_cast<float*>(&tiles[0][0][0][0]) + wq * (DT * 16 + 2) * kWave + lane;
    if (stream == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mg[(dt * 16 + i) * kWave] = st.oacc[dt][i];
      mg[(DT * 16) * kWave] = st.m;
      mg[(DT * 16 + 1) * kWave] = st.l;
    }
    __syncthreads();
    // stream 1's next Q arrives during the merge (this item's Q is done)
    if (stream == 1 && has_next)
      attn_load_q<D>(qf, q, nxt.bh * (int64_t)seq + q_row(nxt), q_row(nxt) < seq, half);
    if (stream == 0) {
      const float m1 = mg[(DT * 16) * kWave], l1 = mg[(DT * 16 + 1) * kWave];
      const float m = fmaxf(st.m, m1);
      const float a0 = __builtin_amdgcn_exp2f(st.m - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.oacc[dt][i] = fmaf(st.oacc[dt][i], a0, mg[(dt * 16 + i) * kWave] * a1);
      st.l = fmaf(st.l, a0, l1 * a1);
      st.m = m;
    }
    // Stream 0 puts the normalised rows in LDS (the last 256*D bytes of the
    // tiles, past the merge area), and all eight waves store them.
    char* otile = reinterpret_cast<char*>(&tiles[0][0][0][0]) + sizeof(tiles) - kAttnBlockM * D * 2;
    static_assert(sizeof(tiles) - kAttnBlockM * D * 2 >= 4 * (DT * 16 + 2) * kWave * sizeof(float),
                  "output tile past the merge area");
    if (stream == 0) attn_row_to_tile<D>(st, otile, wq * 32 + col, lse, base + qi, qi < seq, half);
    // The merge area is the next item's tile memory: every read of it ends
    // here, and the next item's first key blocks are requested right after
    // (the output tile lies in the other stage, which the next item first
    // refills after its own first barrier).
    __syncthreads();
    if (has_next) request_first(nxt);
    attn_store_staged<D, kAttnBlockM, kAttnThreads>(otile, 32 * 2 * D, o, base + qb * kAttnBlockM,
                                                    seq - qb * kAttnBlockM, t);
    // stream 0's next Q, once its merge and rows are done
    if (stream == 0 && has_next)
      attn_load_q<D>(qf, q, nxt.bh * (int64_t)seq + q_row(nxt), q_row(nxt) < seq, half);
    if (!has_next) break;  // uniform over the workgroup
    j = jn;
    cur = nxt;
  }
}

// The same forward with one key stream per workgroup: four waves take the
// 128 queries of one item and walk all its key blocks from the diagonal back,
// with no merge; a workgroup holds half the LDS and two share a compute unit.
// Two independent workgroups per unit hide each other's start-up and
// output stores, which wins when every unit gets many items (long
// sequences); the two-stream kernel halves the longest item's chain, which
// wins when the longest item is a large share of a unit's work.  Workgroup i
// takes item i (heaviest first; on XCD i % 8 with xcd_split).
template <int D>
__global__ __launch_bounds__(kAttnGroupThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attention_fwd_stream_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    uint2* __restrict__ o, float* __restrict__ lse, int seq, int heads, int qblocks, int bh_count,
    bool xcd_split, float scale2, AttnSlopes slopes) {
  constexpr int KS = D / 16;
  constexpr int CH = AttnTile<D>::CHUNKS;
  __shared__ __attribute__((aligned(16))) uint4 tiles[2][2][CH];  // [stage][K, V]

  const int t = threadIdx.x;
  const int w = t / kWave, lane = t & (kWave - 1), half = lane >> 5, col = lane & 31;
  const AttnItem it = attn_item((int)blockIdx.x, qblocks, bh_count, xcd_split);
  const int qb = it.qb;
  const int64_t base = it.bh * (int64_t)seq;
  const float slope2 = slopes.s[(int)(it.bh % heads)];
  const int q0 = qb * kAttnBlockM + w * 32;
  const int qi = q0 + col;
  const bool wave_live = q0 < seq;

  bf16x8_t qf[KS];
  attn_load_q<D>(qf, q, base + qi, qi < seq, half);
  bf16x8_t kx[2];
  attn_key_offsets(kx, half, col);
  const bf16x8_t qx = attn_slope_parts(slope2, scale2, half);
  AttnState<D> st;
  attn_state_init(st);

  const int wg_last_q = min(seq, (qb + 1) * kAttnBlockM) - 1;
  const int nkb = wg_last_q / kAttnBlockN + 1;
  attn_lds_uint4* lt = (attn_lds_uint4*)&tiles[0][0][0];
  auto tile = [&](int stage, int which) { return lt + (stage * 2 + which) * CH; };
  int kb = nkb - 1;
  attn_request<D, false>(k, tile(0, 0), base, kb * kAttnBlockN, seq, w, lane);
  attn_request<D, true>(v, tile(0, 1), base, kb * kAttnBlockN, seq, w, lane);
  attn_wait_loads();
  __syncthreads();
  for (int buf = 0; kb >= 0; buf ^= 1, --kb) {
    const int k0 = kb * kAttnBlockN;
    if (kb >= 1) {
      attn_request<D, false>(k, tile(buf ^ 1, 0), base, k0 - kAttnBlockN, seq, w, lane);
      attn_request<D, true>(v, tile(buf ^ 1, 1), base, k0 - kAttnBlockN, seq, w, lane);
    }
    if (wave_live && k0 <= q0 + 31) {
      if (k0 + kAttnBlockN - 1 > q0)
        attn_block<D, true>(st, tile(buf, 0), tile(buf, 1), qf, kx, qx, scale2, slope2, k0, qi, half, col, lane);
      else
        attn_block<D, false, true>(st, tile(buf, 0), tile(buf, 1), qf, kx, qx, scale2, slope2, k0, qi, half, col,
                                   lane);
    }
    attn_wait_loads();
    __syncthreads();
  }
  // the tiles are free after the last barrier: the rows go through them
  char* otile = reinterpret_cast<char*>(&tiles[0][0][0]);
  static_assert(sizeof(tiles) >= kAttnBlockM * D * 2, "output tile");
  attn_row_to_tile<D>(st, otile, w * 32 + col, lse, base + qi, qi < seq, half);
  __syncthreads();
  attn_store_staged<D, kAttnBlockM, kAttnGroupThreads>(otile, 32 * 2 * D, o, base + qb * kAttnBlockM,
                                                      seq - qb * kAttnBlockM, t);
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
  const int64_t n_items = batch * heads * qblocks;
  const int cus = device_cu_count();
  const int64_t cu8 = (int64_t)(cus / 8) * 8;
  const int64_t g8 = (n_items + 7) / 8 * 8;
  const dim3 grid((unsigned)(g8 < cu8 ? g8 : (cu8 > 0 ? cu8 : 8)));
  // One key stream per workgroup, two workgroups per unit, when a unit's
  // share of the key blocks is at least 1.5x the longest item's (the longest
  // item is the last query block: all its key blocks).  Measured at
  // [1,28,8192,128]: 472.6 against 535.0 us; at [1,28,2048,128]: 54.2 against
  // 44.5 us, where the longest item is two thirds of a unit's share.
  const int64_t nkb_max = (seq - 1) / kAttnBlockN + 1;
  const int64_t blocks_total = (int64_t)batch * heads *
                               [&] {
                                 int64_t t = 0;
                                 for (int qb = 0; qb < qblocks; ++qb)
                                   t += (std::min<int64_t>(seq, (int64_t)(qb + 1) * kAttnBlockM) - 1) / kAttnBlockN + 1;
                                 return t;
                               }();
  const bool one_stream = 2 * blocks_total >= 3 * nkb_max * 2 * (int64_t)(cus > 0 ? cus : 1);
  // whole half-heads per XCD: an even number of query blocks, (b, h) pairs a multiple of 4
  const bool xcd_split = qblocks % 2 == 0 && (batch * heads) % 4 == 0;
  const uint4* qv = reinterpret_cast<const uint4*>(q);
  const uint4* kv = reinterpret_cast<const uint4*>(k);
  const uint4* vv = reinterpret_cast<const uint4*>(v);
  uint2* ov = reinterpret_cast<uint2*>(o);
  const dim3 grid1((unsigned)n_items);
#define BLOOM_ATTN_FWD(DD)                                                                                        \
  if (one_stream)                                                                                                 \
    hipLaunchKernelGGL((attention_fwd_stream_kernel<DD>), grid1, dim3(kAttnGroupThreads), 0, stream, qv, kv, vv, \
                       ov, lse, (int)seq, (int)heads, qblocks, (int)(batch * heads), xcd_split, scale2, table);    \
  else                                                                                                            \
    hipLaunchKernelGGL((attention_fwd_kernel<DD>), grid, dim3(kAttnThreads), 0, stream, qv, kv, vv, ov, lse,      \
                       (int)seq, (int)heads, qblocks, (int)(batch * heads), xcd_split, scale2, table);
  switch (head_dim) {
    case 32:
      BLOOM_ATTN_FWD(32)
      break;
    case 64:
      BLOOM_ATTN_FWD(64)
      break;
    default:
      BLOOM_ATTN_FWD(128)
      break;
  }
#undef BLOOM_ATTN_FWD
  return launch_status("bloom_alibi_attention_fwd");
}
