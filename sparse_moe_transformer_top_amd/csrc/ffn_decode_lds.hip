// Expert gate/up for very small batches (bf16 weights), with the expert's
// token rows in LDS.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section
// "Expert implementation: SwiGLU at scale" (h = silu(x W_gate^T) * (x W_up^T),
// gate and up over the shared input) and section "Tradeoffs" (a handful of
// tokens per expert leaves the layer's cost in reading the expert weights).
//
// With at most 8 tokens, every expert holds at most 8 rows. A work-group
// copies its expert's rows of x into LDS once (rows padded by 16 bytes, so
// the 16 lanes that read one k chunk of 16 rows hit distinct banks) and each
// of its 8 waves then owns one 16-column tile: it streams the tile's 16 gate
// and 16 up weight rows on its own with nontemporal full-line loads (see
// dstep_operands), keeping only weights in flight in its registers
// (kXInFlight double steps of 128 bytes per row), and takes the MFMA
// activation operand from LDS. No cross-wave reduction: a wave's
// accumulators hold its tile's sums over all of H. bf16 weights only: with
// int4 weights (whose conversion and bias MFMAs sit between a wave's load
// batches) the split-k kernel was faster.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kXWaves = 8;        // waves per work-group = column tiles per work-group
constexpr int kXInFlight = 4;     // 128-byte double steps of each weight row in flight per lane
constexpr int kXPad = 8;          // bf16 elements of padding per LDS row

MOE_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__global__ __launch_bounds__(kXWaves * 64) void gateup_xlds_kernel(FfnArgs a) {
  extern __shared__ __align__(16) uint16_t xs[];   // [ne][H + kXPad] bf16
  constexpr int KS = 32;   // k per 64-byte step of a bf16 weight row
  const int tiles = (a.F + 15) / 16;
  const int groups = (tiles + kXWaves - 1) / kXWaves;   // work-groups per expert
  const int e = blockIdx.x / groups;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = (blockIdx.x % groups) * kXWaves + wave;
  const int r0 = a.offsets[e];
  const int ne = a.offsets[e + 1] - r0;
  if (ne <= 0) return;
  const int HP = a.H + kXPad;
  const int i = lane & 15, g = lane >> 4;
  const bool live = tile < tiles;
  const int64_t row_bytes = (int64_t)a.H * 2;
  // this lane's two loads of each double step (dstep_chunk): rows 8h + i % 8
  int64_t woff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = min(min(tile, tiles - 1) * 16 + 8 * h + (i & 7), a.F - 1);
    woff[h] = ((int64_t)e * a.F + n) * row_bytes + 16 * dstep_chunk(h, i, g);
  }
  const char* const wmat[2] = {static_cast<const char*>(a.wg), static_cast<const char*>(a.wu)};
  const int D = a.H / (2 * KS);

  // the expert's token rows into LDS, 16 bytes per thread and pass
  const int cpr = a.H / 8;
  for (int q = threadIdx.x; q < ne * cpr; q += kXWaves * 64) {
    const int r = q / cpr, c = q - r * cpr;
    const int64_t tok = a.perm[r0 + r] / a.k;
    *reinterpret_cast<u32x4*>(xs + r * HP + c * 8) =
        ld16(static_cast<const uint16_t*>(a.x) + tok * a.H + c * 8);
  }
  __syncthreads();
  if (!live) return;

  const bool has_a = i < ne;   // rows past n_e multiply zeros
  const u32x4* const xrow = reinterpret_cast<const u32x4*>(xs + (has_a ? i : 0) * HP);
  const u32x4 z = {0u, 0u, 0u, 0u};
  f32x4 acc[2];
  acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc[1] = acc[0];
  for (int d0 = 0; d0 < D; d0 += kXInFlight) {
    u32x4 bv[kXInFlight][2][2];   // [double step][gate, up][load h]
#pragma unroll
    for (int u = 0; u < kXInFlight; ++u)
      if (d0 + u < D) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            bv[u][b][h] = ld16_nt(wmat[b] + woff[h] + (int64_t)(d0 + u) * 128);
      }
#pragma unroll
    for (int u = 0; u < kXInFlight; ++u) {
      if (d0 + u < D) {
        // this lane group's 8 k of the two 32-k halves: 16-byte chunks
        // 8(d0+u) + g and 8(d0+u) + 4 + g of the activation row
        const u32x4 A0 = has_a ? xrow[8 * (d0 + u) + g] : z;
        const u32x4 A1 = has_a ? xrow[8 * (d0 + u) + 4 + g] : z;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          u32x4 B0, B1;
          dstep_operands(bv[u][b][0], bv[u][b][1], i, B0, B1);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A0), as_bf16x8(B0), acc[b],
                                                           0, 0, 0);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A1), as_bf16x8(B1), acc[b],
                                                           0, 0, 0);
        }
      }
    }
  }

  // 16x16 accumulator layout: lane l holds column l%16, token rows 4*(l/16) + v
  const int col = tile * 16 + i;
  if (col >= a.F) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * g + v;
    if (r >= ne) continue;
    static_cast<uint16_t*>(a.h)[(int64_t)(r0 + r) * a.F + col] =
        f32_to_bf16_bits(swiglu(acc[0][v], acc[1][v]));
  }
}

hipError_t launch_xlds(const FfnArgs& a, size_t lds, hipStream_t s) {
  // allow dynamic LDS beyond the 64 KB default (set on every launch: it is
  // per device, and cheap)
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(gateup_xlds_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kDecodeLdsMax);
  if (err != hipSuccess) return err;
  const int tiles = (a.F + 15) / 16;
  const int groups = (tiles + kXWaves - 1) / kXWaves;
  hipLaunchKernelGGL(gateup_xlds_kernel, dim3((unsigned)(a.E * groups)), dim3(kXWaves * 64), lds,
                     s, a);
  return hipGetLastError();
}

}  // namespace

size_t decode_lds_bytes(int64_t T, int H) {
  return (size_t)T * (size_t)(H + kXPad) * 2;
}

hipError_t launch_gateup_decode_lds(const FfnArgs& a, Wt wt, hipStream_t s) {
  const size_t lds = decode_lds_bytes(a.T, a.H);
  if (wt != WT_BF16 || a.T > kDecodeLdsMaxT || lds > kDecodeLdsMax) return hipErrorNotSupported;
  return launch_xlds(a, lds, s);
}

}  // namespace moe
