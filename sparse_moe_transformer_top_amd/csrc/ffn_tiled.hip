// Expert FFN on the matrix cores: grouped bf16 GEMMs for many rows per expert.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section
// "Expert implementation: SwiGLU at scale": an expert is
// w_down(silu(w_gate x) * w_up x), and gate and up can be fused into one
// product over the shared input (FusedSwiGLUExpert). Kernel 1 computes, for
// each expert, the gate and up tiles of the same output columns in one
// work-group and writes h = silu(g) * u (bf16) from the accumulators; kernel 2
// is the down projection y = h W_down^T.
//
// Both operands are k-contiguous (activation rows [m][k], nn.Linear weights
// [n][k]), so each 16-byte load holds 8 consecutive k of one row, which is the
// per-lane operand of v_mfma_f32_32x32x16_bf16.
//
// Tile: 128 rows x 256 weight rows (gate 128 + up 128, or 256 down columns),
// k in slices of 64; 4 waves in a 2x2 grid, each wave 64 rows x 4 weight
// sub-tiles of 32 (8 MFMA accumulators of 32x32). Slices are staged through
// LDS, double-buffered, with a 16-byte-chunk XOR swizzle so that the 32 lanes
// reading one chunk column of 32 consecutive rows hit distinct banks. The
// activation rows of the gate/up product are gathered from x through the
// dispatch permutation while loading. int8 weights are converted exactly to
// bf16 on their way into LDS; their per-row scales multiply the float32
// accumulators in the epilogue.
#include "common.h"
#include "grouped.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int TBM = 128;  // activation rows per tile
constexpr int TNB = 256;  // weight rows per tile
constexpr int TBK = 64;   // k per LDS stage (8 chunks of 16 bytes per row)

MOE_DEV int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Stage loaders, written as macros so that the per-thread pointer and
// register arrays are indexed only with unrolled constants (and stay in VGPRs).
#define LOAD_GLOBAL(k0)                                                              \
  do {                                                                               \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) ra[i] =                            \
        *reinterpret_cast<const u32x4*>(aptr[i] + (k0));                             \
    _Pragma("unroll") for (int i = 0; i < NBL; ++i) rb[i] =                          \
        *reinterpret_cast<const u32x4*>(bptr[i] + (WT == WT_I8 ? (k0) : 2 * (k0)));  \
  } while (0)

#define STORE_LDS(buf)                                                               \
  do {                                                                               \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                    \
        sA[buf][swz((tid >> 3) + 32 * i, lc)] = ra[i];                               \
    if (WT == WT_I8) {                                                               \
      _Pragma("unroll") for (int i = 0; i < NBL; ++i) {                              \
        const int r_ = (tid >> 2) + 64 * i, c16_ = tid & 3;                          \
        const u32x4 lo_ = i8x8_to_bf16x8(rb[i].x, rb[i].y);                          \
        const u32x4 hi_ = i8x8_to_bf16x8(rb[i].z, rb[i].w);                          \
        sB[buf][swz(r_, 2 * c16_)] = lo_;                                            \
        sB[buf][swz(r_, 2 * c16_ + 1)] = hi_;                                        \
      }                                                                              \
    } else {                                                                         \
      _Pragma("unroll") for (int i = 0; i < NBL; ++i)                                \
          sB[buf][swz((tid >> 3) + 32 * i, lc)] = rb[i];                             \
    }                                                                                \
  } while (0)

template <bool GATEUP, int WT>
__global__ __launch_bounds__(256) void ffn_tiled_kernel(FfnArgs a, uint32_t n_ntiles) {
  __shared__ u32x4 sA[2][TBM * 8];
  __shared__ u32x4 sB[2][TNB * 8];

  GroupedTile tile;
  const uint32_t lin = xcd_swizzle(blockIdx.x, gridDim.x);
  if (!grouped_tile(a.offsets, a.E, TBM, n_ntiles, lin, tile)) return;

  const int N = GATEUP ? a.F : a.H;   // output columns
  const int K = GATEUP ? a.H : a.F;
  constexpr int BNO = GATEUP ? 128 : 256;
  const int n0 = tile.nt * BNO;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = tile.e;

  // ---- global -> register loaders -------------------------------------
  const int lc = tid & 7;  // 16-byte chunk within a 64-wide k slice (bf16)
  const uint16_t* aptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(tile.m0 + (tid >> 3) + 32 * i, tile.m_end - 1);
    if (GATEUP) {
      const int64_t t = a.perm[r] / a.k;
      aptr[i] = static_cast<const uint16_t*>(a.x) + t * a.H + lc * 8;
    } else {
      aptr[i] = static_cast<const uint16_t*>(a.h) + (int64_t)r * a.F + lc * 8;
    }
  }
  constexpr int NBL = WT == WT_I8 ? 4 : 8;  // B loads per thread per stage
  const char* bptr[NBL];
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const int r = WT == WT_I8 ? (tid >> 2) + 64 * i : (tid >> 3) + 32 * i;  // weight row in tile
    const char* base;
    int n;
    if (GATEUP) {
      n = n0 + (r & 127);
      base = static_cast<const char*>(r < 128 ? a.wg : a.wu);
    } else {
      n = n0 + r;
      base = static_cast<const char*>(a.wd);
    }
    n = min(n, N - 1);
    const int64_t elem = ((int64_t)e * N + n) * K;
    if (WT == WT_I8)
      bptr[i] = base + elem + (tid & 3) * 16;
    else
      bptr[i] = base + (elem + lc * 8) * 2;
  }

  u32x4 ra[4], rb[NBL];
  // ---- MFMA main loop -------------------------------------------------
  const int wm = wave >> 1, wn = wave & 1;
  int brow[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    brow[s] = GATEUP ? (s < 2 ? wn * 64 + s * 32 : 128 + wn * 64 + (s - 2) * 32)
                     : wn * 128 + s * 32;
  f32x16 acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][s][v] = 0.f;

  const int KT = K / TBK;
  LOAD_GLOBAL(0);
  STORE_LDS(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) LOAD_GLOBAL((kt + 1) * TBK);
#pragma unroll
    for (int ks = 0; ks < TBK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      bf16x8 af[2], bfv[4];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = as_bf16x8(sA[buf][swz(wm * 64 + mi * 32 + (lane & 31), chunk)]);
#pragma unroll
      for (int s = 0; s < 4; ++s) bfv[s] = as_bf16x8(sB[buf][swz(brow[s] + (lane & 31), chunk)]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[mi][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfv[s], acc[mi][s], 0, 0, 0);
    }
    if (kt + 1 < KT) STORE_LDS(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------
  // 32x32 accumulator layout: lane l holds column l%32; register v holds row
  // 8*(v/4) + 4*(l/32) + v%4.
  const int jcol = lane & 31;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = tile.m0 + wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (r >= tile.m_end) continue;
      if (GATEUP) {
        uint16_t* hrow = static_cast<uint16_t*>(a.h) + (int64_t)r * a.F;
#pragma unroll
        for (int si = 0; si < 2; ++si) {
          const int n = n0 + wn * 64 + si * 32 + jcol;
          if (n >= N) continue;
          float g = acc[mi][si][v], u = acc[mi][si + 2][v];
          if (WT == WT_I8) {
            g *= a.sg[(int64_t)e * a.F + n];
            u *= a.su[(int64_t)e * a.F + n];
          }
          hrow[n] = f32_to_bf16_bits(swiglu(g, u));
        }
      } else {
        uint16_t* yrow = static_cast<uint16_t*>(a.y) + (int64_t)r * a.H;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int n = n0 + wn * 128 + s * 32 + jcol;
          if (n >= N) continue;
          float y = acc[mi][s][v];
          if (WT == WT_I8) y *= a.sd[(int64_t)e * a.H + n];
          yrow[n] = f32_to_bf16_bits(y);
        }
      }
    }
  }
}

template <bool GATEUP, int WT>
hipError_t launch_one(const FfnArgs& a, hipStream_t s) {
  const uint32_t nt = GATEUP ? (uint32_t)((a.F + 127) / 128) : (uint32_t)((a.H + 255) / 256);
  hipLaunchKernelGGL((ffn_tiled_kernel<GATEUP, WT>), dim3(grouped_grid(a.T * a.k, a.E, TBM, nt)),
                     dim3(256), 0, s, a, nt);
  return hipGetLastError();
}

}  // namespace

size_t ffn_ws_bytes(int64_t T, int H, int F, int E, int k, Act act, Wt wt) {
  (void)F; (void)E; (void)wt;
  // the decode path keeps float32 split-k partials of the down projection
  return (act == ACT_BF16 && T <= kDecodeMaxT) ? decode_ws_bytes(T, H, k) : 0;
}

hipError_t launch_gateup_tiled(const FfnArgs& a, Wt wt, hipStream_t s) {
  return wt == WT_I8 ? launch_one<true, WT_I8>(a, s) : launch_one<true, WT_BF16>(a, s);
}

hipError_t launch_down_tiled(const FfnArgs& a, Wt wt, hipStream_t s) {
  return wt == WT_I8 ? launch_one<false, WT_I8>(a, s) : launch_one<false, WT_BF16>(a, s);
}

}  // namespace moe
