// Relative-bias bucket arithmetic shared by every kernel that needs it.
//
// Buckets ("DLRMv4 Brings Sequence-Based Recommendation Training to MLPerf",
// section "Model Architecture": the attention bias depends on positional and
// temporal distance):
//   position: bp = min(max(p(i) - p(j), 0), nP - 1), p(i) = min(i, n_h)
//   time:     bt = min(floor(log2(dt + 1)), nT - 1), dt = min(max(t_i - t_j, 0), 2^31 - 1)
// floor(log2(x)) of x in [1, 2^31] is 31 - clz(x), so the time tables are
// stored indexed by clz: entry c holds the bias of bucket min(31 - c, nT - 1).
#pragma once

#include "common.h"

// Spans of a sequence's timestamps up to this value use the 32-bit path:
// t_i - min + 1 then fits in int32 and dt never reaches the 2^31 - 1 cap.
#define HSTU_NARROW_SPAN_MAX 2147483646LL

// clz index of the time bucket from relative times (narrow path);
// ti1 = (t_i - t_min) + 1, tj = t_j - t_min.
HSTU_DEV int tclz_narrow(int32_t ti1, int32_t tj) {
  int32_t x = ti1 - tj;
  x = x < 1 ? 1 : x;
  return __builtin_clz((uint32_t)x);
}

// clz index from absolute 64-bit times (wide path).
HSTU_DEV int tclz_wide(int64_t ti, int64_t tj) {
  int64_t dt = ti - tj;
  dt = dt < 0 ? 0 : dt;
  dt = dt > 2147483647LL ? 2147483647LL : dt;
  return __builtin_clz((uint32_t)(dt + 1));
}

HSTU_DEV int tbucket_from_clz(int c, int nT) {
  int b = 31 - c;
  return b < nT - 1 ? b : nT - 1;
}

HSTU_DEV int pbucket(int pi, int pj, int nP) {
  int d = pi - pj;
  d = d < 0 ? 0 : d;
  return d < nP - 1 ? d : nP - 1;
}
