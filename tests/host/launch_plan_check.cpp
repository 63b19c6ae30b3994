// Host-only check of the row kernels' launch plans (launch_plan.h) over every
// legal row width and a spread of row counts and compute-unit counts.  A plan
// must give each row a team that covers it with the vectors-per-thread the
// kernel dispatch instantiates (1..8), with no wholly idle vector slot, whole
// teams per workgroup, at most 1024 threads, and a grid that reaches every
// row (forward: one team per row; backward: persistent teams walking rows,
// at most two workgroups per compute unit, since each writes one partial row
// of the column sums).  Prints the number of plans checked; exits 1 on the
// first violation.
#include <cstdio>
#include <cstdlib>

#include "launch_plan.h"

namespace {

int fails = 0;

void fail(const char* what, const char* kind, long long rows, int vecs, int cus, const bloom::RowPlan& p) {
  std::printf("FAIL %s (%s rows=%lld vecs=%d cus=%d): grid=%d block=%d tpr=%d nv=%d\n", what, kind, rows, vecs, cus,
              p.grid, p.block, p.tpr, p.nv);
  if (++fails > 20) std::exit(1);
}

void check_team(const char* kind, long long rows, int vecs, int cus, const bloom::RowPlan& p) {
  if (p.tpr < 64 || p.tpr > 1024 || p.tpr % 64 != 0) fail("team width", kind, rows, vecs, cus, p);
  if (p.nv < 1 || p.nv > 8) fail("vectors per thread outside 1..8", kind, rows, vecs, cus, p);
  if ((long long)p.tpr * p.nv < vecs) fail("team does not cover the row", kind, rows, vecs, cus, p);
  if ((long long)p.tpr * (p.nv - 1) >= vecs) fail("a wholly idle vector slot", kind, rows, vecs, cus, p);
  if (p.block < p.tpr || p.block > 1024 || p.block % p.tpr != 0) fail("workgroup size", kind, rows, vecs, cus, p);
  if (p.grid < 1) fail("empty grid", kind, rows, vecs, cus, p);
}

}  // namespace

int main() {
  const long long row_counts[] = {1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 512, 513,
                                  600, 777, 1000, 2047, 2048, 2049, 4096, 8192, 16384, 100000, 1000003};
  const int cu_counts[] = {1, 4, 80, 104, 228, 256, 304};
  long long checked = 0;
  for (int vecs = 1; vecs <= BLOOM_MAX_HIDDEN / 8; ++vecs) {
    for (long long rows : row_counts) {
      const bloom::RowPlan f = bloom::plan_rows_fwd(rows, vecs);
      check_team("fwd", rows, vecs, 0, f);
      if ((long long)f.grid * (f.block / f.tpr) < rows) fail("forward grid misses rows", "fwd", rows, vecs, 0, f);
      if ((long long)(f.grid - 1) * (f.block / f.tpr) >= rows) fail("forward grid has an idle workgroup", "fwd", rows, vecs, 0, f);
      ++checked;
      for (int cus : cu_counts) {
        const bloom::RowPlan b = bloom::plan_rows_bwd(rows, vecs, cus);
        check_team("bwd", rows, vecs, cus, b);
        if (b.grid > 2 * cus) fail("more than two workgroups per compute unit", "bwd", rows, vecs, cus, b);
        if ((long long)(b.grid - 1) * (b.block / b.tpr) >= rows) fail("backward grid has an idle workgroup", "bwd", rows, vecs, cus, b);
        ++checked;
      }
    }
  }
  std::printf("checked %lld plans, %d failures\n", checked, fails);
  return fails ? 1 : 0;
}
