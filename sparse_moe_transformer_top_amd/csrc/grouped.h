// Grouped-GEMM tile scheduling over the experts' row ranges.
//
// The dispatched rows of expert e are rows offsets[e] .. offsets[e+1]-1. A
// launch covers, per expert, ceil(n_e / BM) row tiles times n_ntiles column
// tiles; the grid is sized on the host for the worst case (ceil(N/BM) + E row
// tiles in total, N = T*k), so no host synchronisation is needed to learn the
// counts, and work-groups past the real tile count exit at once. A launch
// may cover one class of experts (by row count, see in_class). Within an
// expert the row tile varies fastest, so the work-groups sharing one weight
// tile run next to each other (on one XCD, see xcd_tile_index) and read it
// through the same L2.
#pragma once
#include "common.h"

namespace moe {

// Expert classes of a launch: every expert; the experts with at most
// kStreamRows rows (one row tile each of the stream tiles); the experts with
// more.
constexpr int kClsAll = 0;
constexpr int kClsStream = 1;
constexpr int kClsWide = 2;
constexpr int kStreamRows = 128;

MOE_DEV bool in_class(int n, int cls) {
  return cls == kClsAll || (cls == kClsStream ? n <= kStreamRows : n > kStreamRows);
}

// Row tiles of BM rows over expert e's rows [lo, hi) in the launch's class.
MOE_DEV uint32_t class_row_tiles(int lo, int hi, int BM, int cls) {
  const int n = hi - lo;
  return in_class(n, cls) ? (uint32_t)((n + BM - 1) / BM) : 0u;
}

struct GroupedTile {
  int e;        // expert
  int m0;       // first row of the tile
  int m_end;    // one past the expert's last row
  int nt;       // column tile
};

MOE_DEV bool grouped_tile(const int32_t* __restrict__ offsets, int E, int BM, uint32_t n_ntiles,
                          int cls, uint32_t lin, GroupedTile& out) {
  int lo = offsets[0];
  for (int e = 0; e < E; ++e) {
    const int hi = offsets[e + 1];
    const uint32_t mt = class_row_tiles(lo, hi, BM, cls);
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
                            uint32_t n_ntiles, int cls, uint32_t& lin) {
  uint32_t R = 0;
  for (int e = 0; e < E; ++e) R += class_row_tiles(offsets[e], offsets[e + 1], BM, cls) * n_ntiles;
  const uint32_t per = (R + 7) / 8, slot = blockIdx.x >> 3;
  if (slot >= per) return false;
  lin = (blockIdx.x & 7) * per + slot;
  return true;
}

// Tail split. With one work-group per CU, an XCD's tiles run in rounds of
// kCusPerXcd; when its count is not a multiple of that, the last round is
// partial and most of the XCD waits for it. Those tail tiles are cut along k
// into S pieces each (tail_pieces), so the tail takes ceil(tail S /
// kCusPerXcd) rounds of 1/S of a tile instead of one whole tile. Pieces write
// float32 partial tiles to scratch slot (xcd, q) (q = slot - full, below
// kTailSlots); a reduce kernel adds them in piece order. Work items of one
// XCD: slots [0, full) are whole tiles, slots full + j*S + p are piece p of
// tail tile j.
constexpr int kCusPerXcd = 32;             // MI355X: 256 CUs in 8 XCDs
constexpr uint32_t kTailSlots = 96;        // partial tiles per XCD in scratch
constexpr uint32_t kTailMaxPieces = 8;

// Pieces per tail tile: over S <= min(kTailMaxPieces, max_pieces) with
// tail * S <= kTailSlots, the S whose pieces finish first (ceil(tail S / 32)
// / S of a tile), a larger S taken only for a gain of 10% or more over the
// best smaller one (each piece adds a partial tile to write and read back).
// 12 tail tiles: 5 pieces (0.4 of a tile); 24: 4 pieces (0.75).
MOE_DEV uint32_t tail_pieces(uint32_t tail, uint32_t max_pieces) {
  uint32_t best = 1, rounds = 1;   // the best time is rounds / best tiles
  for (uint32_t S = 2; S <= kTailMaxPieces && S <= max_pieces && S * tail <= kTailSlots; ++S) {
    const uint32_t r = (tail * S + kCusPerXcd - 1) / kCusPerXcd;
    if (10 * r * best < 9 * rounds * S) {
      best = S;
      rounds = r;
    }
  }
  return best;
}

struct TailPlan {
  uint32_t base;   // first real tile of this XCD
  uint32_t full;   // whole tiles before the tail
  uint32_t tail;   // tail tiles
  uint32_t S;      // pieces per tail tile (1: the tail is not split)
};

MOE_DEV TailPlan tail_plan(const int32_t* __restrict__ offsets, int E, int BM, uint32_t n_ntiles,
                           int cls, uint32_t xcd, int max_pieces) {
  uint32_t R = 0;
  for (int e = 0; e < E; ++e) R += class_row_tiles(offsets[e], offsets[e + 1], BM, cls) * n_ntiles;
  const uint32_t per = (R + 7) / 8;
  TailPlan t;
  t.base = xcd * per;
  const uint32_t cnt = R > t.base ? min(per, R - t.base) : 0u;
  t.full = cnt / kCusPerXcd * kCusPerXcd;
  t.tail = cnt - t.full;
  t.S = t.tail ? tail_pieces(t.tail, (uint32_t)max_pieces) : 1u;
  return t;
}

// This work-group's item: tile index lin, and piece (-1 for a whole tile) of
// npieces, with its scratch slot. False for work-groups past the work.
MOE_DEV bool xcd_tail_work(const int32_t* __restrict__ offsets, int E, int BM,
                           uint32_t n_ntiles, int cls, int max_pieces, uint32_t& lin, int& piece,
                           int& npieces, uint32_t& slot_out) {
  const uint32_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const TailPlan t = tail_plan(offsets, E, BM, n_ntiles, cls, xcd, max_pieces);
  if (slot < t.full) {
    lin = t.base + slot;
    piece = -1;
    npieces = 1;
    return true;
  }
  const uint32_t q = slot - t.full;
  if (q >= t.tail * t.S) return false;
  lin = t.base + t.full + q / t.S;
  npieces = (int)t.S;
  piece = t.S > 1 ? (int)(q % t.S) : -1;
  slot_out = xcd * kTailSlots + q;
  return true;
}

// Extra work-groups a tail-split launch may need beyond the tile grid: per
// XCD, full + tail S <= (its tiles) + kTailSlots.
constexpr unsigned kTailExtraBlocks = 8 * kTailSlots;
// Float32 partial tiles of the split pieces (one tile of up to 256 x 256
// elements per slot).
constexpr size_t kTailScratchBytes = (size_t)8 * kTailSlots * 256 * 256 * 4;

// Worst-case grid, a multiple of 8 (see xcd_tile_index).
inline unsigned grouped_grid(int64_t n_assign, int E, int BM, int n_ntiles) {
  const int64_t mt = (n_assign + BM - 1) / BM + E;
  return (unsigned)((mt * n_ntiles + 7) / 8 * 8);
}

}  // namespace moe
