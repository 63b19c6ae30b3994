// Launch shapes of the row kernels and the shared column-sum launcher.
//
// A row of `vecs` 16-byte vectors is owned by a team of `tpr` threads, each
// holding `nv` vectors (vector v = t + k*tpr).  Narrow rows (<= 512 vectors,
// i.e. H <= 4096) use one wave64 per row; wider rows use a whole workgroup of
// up to 1024 threads, sized so that nv <= nv_cap with as few idle lanes as
// possible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bloom_kernels.h"

namespace bloom {

struct RowPlan {
  int grid;   // workgroups
  int block;  // threads per workgroup
  int tpr;    // threads per row team (64 = wave mode)
  int nv;     // 16-byte vectors per thread (template parameter, 1..8)
};

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Team width for a row of `vecs` vectors with at most nv_cap vectors per
// thread: as few idle lanes as possible, and among equally good widths the
// widest team (fewest vectors per thread: lower register use, more waves in
// flight per compute unit).  A row too wide for the cap even at 1024 threads
// gets the widest team with as few vectors per thread as cover it.
inline void pick_team(int vecs, int nv_cap, int& tpr, int& nv) {
  if (vecs <= 64 * nv_cap) {
    tpr = 64;
    nv = ceil_div(vecs, 64);
    return;
  }
  int best_w = 16, best_waste = 1 << 30, best_nv = ceil_div(vecs, 1024);
  for (int w = 16; w >= 2; --w) {
    const int t = 64 * w;
    const int n = ceil_div(vecs, t);
    if (n > nv_cap) continue;
    const int waste = t * n - vecs;
    if (waste < best_waste) {
      best_waste = waste;
      best_w = w;
      best_nv = n;
    }
  }
  tpr = 64 * best_w;
  nv = best_nv;
}

// Forward team: as few idle lanes as possible, and among equally good widths
// the NARROWEST (most vectors per thread).  The forward holds only its own row
// in registers, so the bytes a compute unit keeps in flight grow with the
// vectors per thread faster than the register cost cuts the resident waves
// (e.g. H = 14336: 256 threads x 7 vectors keeps ~140 KB per CU in flight,
// 896 x 2 only ~64 KB).
inline void pick_team_narrow(int vecs, int nv_cap, int& tpr, int& nv) {
  if (vecs <= 64 * nv_cap) {
    tpr = 64;
    nv = ceil_div(vecs, 64);
    return;
  }
  int best_w = 16, best_waste = 1 << 30, best_nv = ceil_div(vecs, 1024);
  for (int w = 2; w <= 16; ++w) {
    const int t = 64 * w;
    const int n = ceil_div(vecs, t);
    if (n > nv_cap) continue;
    const int waste = t * n - vecs;
    if (waste < best_waste) {
      best_waste = waste;
      best_w = w;
      best_nv = n;
    }
  }
  tpr = 64 * best_w;
  nv = best_nv;
}

inline RowPlan plan_rows_fwd(int64_t rows, int vecs) {
  RowPlan p;
  pick_team_narrow(vecs, 8, p.tpr, p.nv);
  if (p.tpr == 64) {
    p.block = 256;
    p.grid = ceil_div(rows, p.block / 64);
  } else {
    p.block = p.tpr;
    p.grid = (int)rows;
  }
  return p;
}

// Backward: one workgroup per compute unit at most (the column partial rows
// it writes scale with the grid; two for H = 2048, below), teams walk rows
// with stride grid*teams.
inline RowPlan plan_rows_bwd(int64_t rows, int vecs, int cus) {
  RowPlan p;
  pick_team(vecs, 4, p.tpr, p.nv);
  if (vecs == 256) {
    // H = 2048: a four-wave team per row, one vector per thread (the streaming
    // kernel), two workgroups per compute unit.  The wave-per-row form holds a
    // row's 32 elements per lane at 210 registers, two waves per SIMD, and its
    // arithmetic per wave is then as long as its memory time.  Measured at
    // [8192, 2048]: 46.2 -> 29.9 us; [16384, 2048] 64.1 -> 47.3; [2048, 2048]
    // 22.6 -> 15.4 (one workgroup per unit: 40.4, 72.0, 16.3; four: 31.1,
    // 48.4, 18.3).
    p.tpr = 256;
    p.nv = 1;
    p.block = p.tpr;
    const int64_t g = (int64_t)cus * 2;
    p.grid = (int)(rows < g ? rows : g);
    if (p.grid < 1) p.grid = 1;
    return p;
  }
  if (p.tpr == 64) {
    // A wave per row: eight rows in flight per workgroup (the eight waves'
    // column sums are added in LDS, still one partial row per workgroup)
    // when each wave gets at least two rows, else four.  Measured at
    // [8192, 2048]: 36.5 -> 32.3 us; with one row per wave ([2048, 2048])
    // four waves were 3 % faster.
    p.block = rows >= (int64_t)cus * 16 ? 512 : 256;
    const int teams = p.block / 64;
    p.grid = ceil_div(rows, teams);
  } else {
    p.block = p.tpr;
    p.grid = (int)rows;
  }
  if (p.grid > cus) p.grid = cus;
  if (p.grid < 1) p.grid = 1;
  return p;
}

// Instantiates CALL(NV, MAXB) for the plan: NV = vectors per thread, MAXB =
// the launch bound (256, 512 or 1024) that covers p.block, so a kernel built
// for small workgroups may use the larger register budget they allow.
#define BLOOM_ROW_DISPATCH_NV(nv, MAXB, CALL) \
  switch (nv) {                               \
    case 1: CALL(1, MAXB); break;             \
    case 2: CALL(2, MAXB); break;             \
    case 3: CALL(3, MAXB); break;             \
    case 4: CALL(4, MAXB); break;             \
    case 5: CALL(5, MAXB); break;             \
    case 6: CALL(6, MAXB); break;             \
    case 7: CALL(7, MAXB); break;             \
    default: CALL(8, MAXB); break;            \
  }
#define BLOOM_ROW_DISPATCH(p, CALL)                  \
  do {                                               \
    if ((p).block <= 256) {                          \
      BLOOM_ROW_DISPATCH_NV((p).nv, 256, CALL)       \
    } else if ((p).block <= 512) {                   \
      BLOOM_ROW_DISPATCH_NV((p).nv, 512, CALL)       \
    } else {                                         \
      BLOOM_ROW_DISPATCH_NV((p).nv, 1024, CALL)      \
    }                                                \
  } while (0)

// Sums `parts` partial rows of `cols` fp32 columns (row-major [parts][cols])
// in row order and writes bf16: columns [0, split) to out0, [split, cols) to
// out1 (out1 may be NULL when split == cols).
void launch_colsum(const float* partial, int parts, int64_t cols, int64_t split, bloom_bf16* out0,
                   bloom_bf16* out1, hipStream_t stream);

}  // namespace bloom
