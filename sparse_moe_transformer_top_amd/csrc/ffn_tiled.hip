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
// bf16 weights (ffn_mfma_kernel): a work-group of 8 waves computes a tile of
// 256 activation rows x 256 weight rows (gate 128 + up 128, or 256 down
// columns); waves form a 4 x 2 grid, each wave 64 rows x 4 weight sub-tiles
// of 32 (8 MFMA accumulators of 32x32, two waves per SIMD). k advances in
// slices of 64 through a two-stage LDS ring filled by direct global->LDS
// loads (global_load_lds_dwordx4, no register staging); the activation rows
// of the gate/up product are gathered from x through the dispatch permutation
// by the addresses of those loads. Each wave loads its MFMA operands for the
// next 16-k step while the current step's MFMAs run, across the stage
// boundary as well, and the scheduler is asked to issue one LDS read after
// each MFMA. LDS rows use a 16-byte-chunk XOR swizzle so the 32 lanes reading
// one chunk column of 32 consecutive rows hit distinct banks.
//
// int8 weights (ffn_tiled_kernel): 128 x 256 tiles of 4 waves, staged through
// registers so that the weights can be converted exactly to bf16 on their way
// into LDS; per-row scales multiply the float32 accumulators in the epilogue.
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


// ---------------------------------------------------------------------------
// bf16 weights: direct-to-LDS pipelined kernel
// ---------------------------------------------------------------------------
constexpr int MBM = 256;   // activation rows per tile
constexpr int MNB = 256;   // weight rows per tile
constexpr int MBK = 64;    // k per LDS stage
constexpr int MWM = 4, MWN = 2, MNW = MWM * MWN;   // wave grid
constexpr int MLPW = MBM * 8 / 64 / MNW;           // LDS-DMA loads per wave per operand per stage

typedef __attribute__((address_space(3))) void lds_void_t;

// 64 lanes x 16 bytes from per-lane global addresses into LDS at l + 16*lane
// (l wave-uniform). Written as asm because the compiler's wait-count pass,
// unable to tell the two LDS stages apart, otherwise drains every outstanding
// load before each LDS read; this kernel places its own vmcnt waits. The load
// writes no VGPR.
MOE_DEV void lds_dma16(const void* g, void* l) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void_t*)l;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}

// s_waitcnt vmcnt(N) leaving the other counters untouched
template <int N>
MOE_DEV void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
MOE_DEV void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// work-group barrier that the compiler may not move memory operations across
MOE_DEV void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool GATEUP>
__global__ __launch_bounds__(MNW * 64) void ffn_mfma_kernel(FfnArgs a, uint32_t n_ntiles) {
  constexpr int CH = MBK / 8;                 // 16-byte chunks per LDS row
  constexpr int MW = MBM / MWM, NWR = MNB / MWN;
  constexpr int MI = MW / 32, NI = NWR / 32;  // 2 x 4 accumulators
  constexpr int NKS = MBK / 16;
  // one LDS variable per stage: the A tile then the B tile
  __shared__ u32x4 sT0[(MBM + MNB) * CH], sT1[(MBM + MNB) * CH];
  u32x4* const SA[2] = {sT0, sT1};
  u32x4* const SB[2] = {sT0 + MBM * CH, sT1 + MBM * CH};

  GroupedTile tile;
  const uint32_t lin = xcd_swizzle(blockIdx.x, gridDim.x);
  if (!grouped_tile(a.offsets, a.E, MBM, n_ntiles, lin, tile)) return;
  const int N = GATEUP ? a.F : a.H;
  const int K = GATEUP ? a.H : a.F;
  constexpr int BNO = GATEUP ? MNB / 2 : MNB;  // output columns per tile
  const int n0 = tile.nt * BNO;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, e = tile.e;

  // LDS chunk q of a stage holds row q / CH, physical chunk q % CH, which is
  // logical k-chunk (q % CH) ^ ((row >> 1) & 7)
  const uint16_t* asrc[MLPW];
  const uint16_t* bsrc[MLPW];
#pragma unroll
  for (int j = 0; j < MLPW; ++j) {
    const int q = (MLPW * wave + j) * 64 + lane;
    const int r = q / CH, c = (q % CH) ^ ((r >> 1) & 7);
    const int row = min(tile.m0 + r, tile.m_end - 1);
    if (GATEUP)
      asrc[j] = static_cast<const uint16_t*>(a.x) + (int64_t)(a.perm[row] / a.k) * a.H + c * 8;
    else
      asrc[j] = static_cast<const uint16_t*>(a.h) + (int64_t)row * a.F + c * 8;
    int n;
    const uint16_t* base;
    if (GATEUP) {
      n = n0 + (r & (MNB / 2 - 1));
      base = static_cast<const uint16_t*>(r < MNB / 2 ? a.wg : a.wu);
    } else {
      n = n0 + r;
      base = static_cast<const uint16_t*>(a.wd);
    }
    n = min(n, N - 1);
    bsrc[j] = base + ((int64_t)e * N + n) * K + c * 8;
  }

  const int wm = wave / MWN, wn = wave % MWN;
  int arow[MI], brow[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) arow[mi] = wm * MW + mi * 32 + (lane & 31);
#pragma unroll
  for (int s = 0; s < NI; ++s)
    brow[s] = (GATEUP ? (s < NI / 2 ? wn * (NWR / 2) + s * 32
                                    : MNB / 2 + wn * (NWR / 2) + (s - NI / 2) * 32)
                      : wn * NWR + s * 32) + (lane & 31);
  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int s = 0; s < NI; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][s][v] = 0.f;
  bf16x8 fa[2][MI], fb[2][NI];

#define MOE_ISSUE(ST, K0)                                              \
  do {                                                                 \
    _Pragma("unroll") for (int j = 0; j < MLPW; ++j) {                 \
      lds_dma16(asrc[j] + (K0), SA[ST] + (MLPW * wave + j) * 64);      \
      lds_dma16(bsrc[j] + (K0), SB[ST] + (MLPW * wave + j) * 64);      \
    }                                                                  \
  } while (0)
#define MOE_LOADF(SLOT, ST, KS)                                                        \
  do {                                                                                 \
    const int chunk_ = (KS) * 2 + (lane >> 5);                                         \
    _Pragma("unroll") for (int mi = 0; mi < MI; ++mi) fa[SLOT][mi] = as_bf16x8(        \
        SA[ST][arow[mi] * CH + (chunk_ ^ ((arow[mi] >> 1) & 7))]);                     \
    _Pragma("unroll") for (int s = 0; s < NI; ++s) fb[SLOT][s] = as_bf16x8(            \
        SB[ST][brow[s] * CH + (chunk_ ^ ((brow[s] >> 1) & 7))]);                       \
  } while (0)

  const int KT = K / MBK;
  MOE_ISSUE(0, 0);
  if (KT > 1) MOE_ISSUE(1, MBK);
  if (KT > 1) wait_vmcnt<2 * MLPW>(); else wait_vmcnt<0>();
  block_sync();
  MOE_LOADF(0, 0, 0);
  for (int kt0 = 0; kt0 < KT; kt0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kt = kt0 + u;
      if (kt < KT) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int slot = ks & 1;
          if (ks + 1 < NKS) {
            MOE_LOADF(slot ^ 1, u, ks + 1);
          } else if (kt + 1 < KT) {
            // stage kt+1 landed for every wave and nobody reads stage kt any
            // more: refill stage kt's buffer with stage kt+2
            wait_vmcnt<0>();
            wait_lgkmcnt0();
            block_sync();
            if (kt + 2 < KT) MOE_ISSUE(u, (kt + 2) * MBK);
            MOE_LOADF(slot ^ 1, u ^ 1, 0);
          }
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int s = 0; s < NI; ++s)
              acc[mi][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][mi], fb[slot][s],
                                                                   acc[mi][s], 0, 0, 0);
          // one MFMA, then one LDS read of the next step's operands
#pragma unroll
          for (int q = 0; q < MI * NI; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (q < MI + NI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
      }
    }
  }
#undef MOE_ISSUE
#undef MOE_LOADF

  // epilogue; 32x32 accumulator layout: lane l holds column l%32, register
  // v holds row 8*(v/4) + 4*(l/32) + v%4
  const int jcol = lane & 31;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = tile.m0 + wm * MW + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (r >= tile.m_end) continue;
      if (GATEUP) {
        uint16_t* hrow = static_cast<uint16_t*>(a.h) + (int64_t)r * a.F;
#pragma unroll
        for (int si = 0; si < NI / 2; ++si) {
          const int n = n0 + wn * (NWR / 2) + si * 32 + jcol;
          if (n < N) hrow[n] = f32_to_bf16_bits(swiglu(acc[mi][si][v], acc[mi][si + NI / 2][v]));
        }
      } else {
        uint16_t* yrow = static_cast<uint16_t*>(a.y) + (int64_t)r * a.H;
#pragma unroll
        for (int s = 0; s < NI; ++s) {
          const int n = n0 + wn * NWR + s * 32 + jcol;
          if (n < N) yrow[n] = f32_to_bf16_bits(acc[mi][s][v]);
        }
      }
    }
  }
}

template <bool GATEUP>
hipError_t launch_mfma(const FfnArgs& a, hipStream_t s) {
  const uint32_t nt = GATEUP ? (uint32_t)((a.F + MNB / 2 - 1) / (MNB / 2))
                             : (uint32_t)((a.H + MNB - 1) / MNB);
  hipLaunchKernelGGL((ffn_mfma_kernel<GATEUP>), dim3(grouped_grid(a.T * a.k, a.E, MBM, nt)),
                     dim3(MNW * 64), 0, s, a, nt);
  return hipGetLastError();
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
  return wt == WT_I8 ? launch_one<true, WT_I8>(a, s) : launch_mfma<true>(a, s);
}

hipError_t launch_down_tiled(const FfnArgs& a, Wt wt, hipStream_t s) {
  return wt == WT_I8 ? launch_one<false, WT_I8>(a, s) : launch_mfma<false>(a, s);
}

}  // namespace moe
