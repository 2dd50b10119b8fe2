// Expert FFN, float32 activations and weights (grouped over experts).
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section
// "Expert implementation: SwiGLU at scale": each expert computes
// w_down(silu(w_gate x) * w_up x); gate and up share their input and are
// computed together (the page's fused gate/up form), with silu(g)*u applied
// in the epilogue of that product.
//
// Plain LDS-tiled VALU GEMM (64x64 tile, 16-deep k slices, 4x4 outputs per
// thread); float32 FMA accumulation in k order. This path serves the small
// float32 workloads; the bf16 path runs on the matrix cores.
#include "common.h"
#include "grouped.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 64, BN = 64, BK = 16;

template <bool GATEUP>
__global__ __launch_bounds__(256) void ffn_f32_kernel(FfnArgs a, uint32_t n_ntiles) {
  constexpr int NB = GATEUP ? 2 : 1;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[NB][BK][BN + 4];
  GroupedTile tile;
  if (!grouped_tile(a.offsets, a.E, BM, n_ntiles, kClsAll, blockIdx.x, tile)) return;
  const int N = GATEUP ? a.F : a.H;
  const int K = GATEUP ? a.H : a.F;
  const int n0 = tile.nt * BN;
  const int tid = threadIdx.x;

  // loader: 64 rows x 16 k = 256 float4 -> one float4 per thread per matrix
  const int lr = tid >> 2, lc = (tid & 3) * 4;
  const int arow = min(tile.m0 + lr, tile.m_end - 1);
  const float* aptr;
  if (GATEUP) {
    const int64_t t = a.perm[arow] / a.k;
    aptr = static_cast<const float*>(a.x) + t * a.H;
  } else {
    aptr = static_cast<const float*>(a.h) + (int64_t)arow * a.F;
  }
  const int bn = min(n0 + lr, N - 1);
  const float* bptr[NB];
  if (GATEUP) {
    bptr[0] = static_cast<const float*>(a.wg) + ((int64_t)tile.e * a.F + bn) * a.H;
    bptr[NB - 1] = static_cast<const float*>(a.wu) + ((int64_t)tile.e * a.F + bn) * a.H;
  } else {
    bptr[0] = static_cast<const float*>(a.wd) + ((int64_t)tile.e * a.H + bn) * a.F;
  }

  const int ty = tid >> 4, tx = tid & 15;
  float acc[NB][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    const float4 av = *reinterpret_cast<const float4*>(aptr + k0 + lc);
    As[lc + 0][lr] = av.x; As[lc + 1][lr] = av.y; As[lc + 2][lr] = av.z; As[lc + 3][lr] = av.w;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float4 bv = *reinterpret_cast<const float4*>(bptr[b] + k0 + lc);
      Bs[b][lc + 0][lr] = bv.x; Bs[b][lc + 1][lr] = bv.y;
      Bs[b][lc + 2][lr] = bv.z; Bs[b][lc + 3][lr] = bv.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float ar[4], br[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) br[b][j] = Bs[b][kk][tx * 4 + j];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(ar[i], br[b][j], acc[b][i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tile.m0 + ty * 4 + i;
    if (r >= tile.m_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      if (GATEUP)
        static_cast<float*>(a.h)[(int64_t)r * a.F + n] = swiglu(acc[0][i][j], acc[NB - 1][i][j]);
      else
        static_cast<float*>(a.y)[(int64_t)r * a.H + n] = acc[0][i][j];
    }
  }
}

}  // namespace

hipError_t launch_gateup_f32(const FfnArgs& a, hipStream_t s) {
  const uint32_t nt = (uint32_t)((a.F + BN - 1) / BN);
  hipLaunchKernelGGL(ffn_f32_kernel<true>, dim3(grouped_grid(a.T * a.k, a.E, BM, nt)), dim3(256),
                     0, s, a, nt);
  return hipGetLastError();
}

hipError_t launch_down_f32(const FfnArgs& a, hipStream_t s) {
  const uint32_t nt = (uint32_t)((a.H + BN - 1) / BN);
  hipLaunchKernelGGL(ffn_f32_kernel<false>, dim3(grouped_grid(a.T * a.k, a.E, BM, nt)), dim3(256),
                     0, s, a, nt);
  return hipGetLastError();
}

}  // namespace moe
