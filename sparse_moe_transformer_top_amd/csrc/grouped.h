// Grouped-GEMM tile scheduling over the experts' row ranges.
//
// The dispatched rows of expert e are rows offsets[e] .. offsets[e+1]-1. A
// launch covers, per expert, ceil(n_e / BM) row tiles times n_ntiles column
// tiles; the grid is sized on the host for the worst case (ceil(N/BM) + E row
// tiles in total, N = T*k), so no host synchronisation is needed to learn the
// counts, and work-groups past the real tile count exit at once. Within an
// expert the row tile varies fastest, so the work-groups sharing one weight
// tile run next to each other (on one XCD after xcd_swizzle) and read it
// through the same L2.
#pragma once
#include "common.h"

namespace moe {

struct GroupedTile {
  int e;        // expert
  int m0;       // first row of the tile
  int m_end;    // one past the expert's last row
  int nt;       // column tile
};

MOE_DEV bool grouped_tile(const int32_t* __restrict__ offsets, int E, int BM, uint32_t n_ntiles,
                          uint32_t lin, GroupedTile& out) {
  int lo = offsets[0];
  for (int e = 0; e < E; ++e) {
    const int hi = offsets[e + 1];
    const uint32_t mt = (uint32_t)((hi - lo + BM - 1) / BM);
    const uint32_t cnt = mt * n_ntiles;
    if (lin < cnt) {
      out.e = e;
      out.nt = (int)(lin / mt);
      out.m0 = lo + (int)(lin % mt) * BM;
      out.m_end = hi;
      return true;
    }
    lin -= cnt;
    lo = hi;
  }
  return false;
}

inline unsigned grouped_grid(int64_t n_assign, int E, int BM, int n_ntiles) {
  const int64_t mt = (n_assign + BM - 1) / BM + E;
  return (unsigned)(mt * n_ntiles);
}

}  // namespace moe
