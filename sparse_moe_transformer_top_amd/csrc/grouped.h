// Grouped-GEMM tile scheduling over the experts' row ranges.
//
// The dispatched rows of expert e are rows offsets[e] .. offsets[e+1]-1. A
// launch covers, per expert, ceil(n_e / BM) row tiles times n_ntiles column
// tiles; the grid is sized on the host for the worst case (ceil(N/BM) + E row
// tiles in total, N = T*k), so no host synchronisation is needed to learn the
// counts, and work-groups past the real tile count exit at once. Within an
// expert the row tile varies fastest, so the work-groups sharing one weight
// tile run next to each other (on one XCD, see xcd_tile_index) and read it
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

// XCD-balanced tile index. Work-group b runs on XCD b % 8 (the dispatcher
// deals work-groups to the 8 XCDs in turn). The R real tiles are split into 8
// contiguous ranges of ceil(R/8), one per XCD, so that tiles sharing operands
// meet in one L2 and every XCD gets the same number of tiles (a grid sized
// for the worst case would otherwise leave the surplus on the last XCDs).
// Work-groups past the end return false; grouped_tile() rejects an index past
// R on the last XCD.
MOE_DEV bool xcd_tile_index(const int32_t* __restrict__ offsets, int E, int BM,
                            uint32_t n_ntiles, uint32_t& lin) {
  uint32_t R = 0;
  for (int e = 0; e < E; ++e)
    R += (uint32_t)((offsets[e + 1] - offsets[e] + BM - 1) / BM) * n_ntiles;
  const uint32_t per = (R + 7) / 8, slot = blockIdx.x >> 3;
  if (slot >= per) return false;
  lin = (blockIdx.x & 7) * per + slot;
  return true;
}

// Worst-case grid, a multiple of 8 (see xcd_tile_index).
inline unsigned grouped_grid(int64_t n_assign, int E, int BM, int n_ntiles) {
  const int64_t mt = (n_assign + BM - 1) / BM + E;
  return (unsigned)((mt * n_ntiles + 7) / 8 * 8);
}

}  // namespace moe
