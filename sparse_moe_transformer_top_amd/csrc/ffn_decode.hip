// Expert FFN for few rows per expert (decode): weight streaming.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section
// "Expert implementation: SwiGLU at scale" (w_down(silu(w_gate x) * w_up x),
// gate and up fused over the shared input) and section "Tradeoffs" (small
// expert batches leave the matrix units idle: with a handful of tokens per
// expert the layer's cost is reading the experts' weights once).
//
// With at most 16 rows per expert every weight element is used by <= 16 rows,
// so the kernels are bound by HBM: the goal is to stream each touched
// expert's weights exactly once at full bandwidth, and nothing else. A
// work-group owns 16 weight rows of one expert (gate and up rows of the same
// 16 output columns for kernel 1, 16 down rows for kernel 2) and splits k
// across its 4 waves; each lane keeps kInFlight independent 16-byte weight
// loads outstanding. The products run on v_mfma_f32_16x16x32_bf16 with the
// expert's rows as the 16-row A operand (rows past n_e are zero). The 4
// waves' partial sums are added in wave order through LDS. int8 weights are
// loaded 16 per lane (64 k per step) and converted exactly to bf16; their
// row scales multiply the float32 sums.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kInFlight = 8;

typedef float f32x4v __attribute__((ext_vector_type(4)));

MOE_DEV uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// One k step of one lane: A (activation) operand(s) and B (weight) operand(s).
// bf16 weights: 32 k per step, one A and one B operand.
// int8 weights: 64 k per step, two A operands (32 contiguous bytes of the
// row), one 16-byte int8 load split into two B operands.
template <int WT>
struct Step {
  static constexpr int K = WT == WT_I8 ? 64 : 32;
};

template <int WT, int NB>
MOE_DEV void mfma_step(const uint4 (&av)[2], const uint4 (&bv)[NB], f32x4v (&acc)[NB]) {
  if (WT == WT_I8) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      uint4 lo, hi;
      i8x4_to_bf16x4(bv[b].x, lo.x, lo.y);
      i8x4_to_bf16x4(bv[b].y, lo.z, lo.w);
      i8x4_to_bf16x4(bv[b].z, hi.x, hi.y);
      i8x4_to_bf16x4(bv[b].w, hi.z, hi.w);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[0]), as_bf16x8(lo), acc[b], 0,
                                                       0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[1]), as_bf16x8(hi), acc[b], 0,
                                                       0, 0);
    }
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[0]), as_bf16x8(bv[b]), acc[b],
                                                       0, 0, 0);
  }
}

// Stream NB weight matrices' rows [n0, n0+16) (row length K) against the
// A rows arow (nullptr for a zero row). Returns this wave's partial sums.
template <int WT, int NB>
MOE_DEV void stream_rows(const uint16_t* arow, const char* const (&wrow)[NB], int K, int wave,
                         int g, f32x4v (&acc)[NB]) {
  constexpr int KS = Step<WT>::K;
  constexpr int ESZ = WT == WT_I8 ? 1 : 2;
  const int nsteps = K / KS;
  for (int s0 = wave; s0 < nsteps; s0 += kWaves * kInFlight) {
    uint4 bv[kInFlight][NB];
    uint4 av[kInFlight][2];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int s = s0 + kWaves * u;
      if (s < nsteps) {
        const int k0 = s * KS;
        const int kl = WT == WT_I8 ? 16 * g : 8 * g;  // this lane's first k within the step
#pragma unroll
        for (int b = 0; b < NB; ++b) bv[u][b] = ldg16(wrow[b] + (int64_t)(k0 + kl) * ESZ);
        const uint4 z = make_uint4(0, 0, 0, 0);
        av[u][0] = arow ? ldg16(arow + k0 + kl) : z;
        av[u][1] = (WT == WT_I8 && arow) ? ldg16(arow + k0 + kl + 8) : z;
      }
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      if (s0 + kWaves * u < nsteps) mfma_step<WT, NB>(av[u], bv[u], acc);
    }
  }
}

// Kernel 1: h = silu(x W_gate^T) * (x W_up^T) for <= 16 rows per expert.
template <int WT>
__global__ __launch_bounds__(kWaves * 64) void gateup_decode_kernel(FfnArgs a) {
  __shared__ float red[kWaves][2][4][64];
  const int nt_per_e = (a.F + 15) / 16;
  const int e = blockIdx.x / nt_per_e;
  const int n0 = (blockIdx.x % nt_per_e) * 16;
  const int r0 = a.offsets[e];
  const int ne = a.offsets[e + 1] - r0;
  if (ne <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const uint16_t* arow = nullptr;
  if (i < ne) arow = static_cast<const uint16_t*>(a.x) + (int64_t)(a.perm[r0 + i] / a.k) * a.H;
  const int n = min(n0 + i, a.F - 1);
  constexpr int ESZ = WT == WT_I8 ? 1 : 2;
  const int64_t roff = ((int64_t)e * a.F + n) * a.H * ESZ;
  const char* const wrow[2] = {static_cast<const char*>(a.wg) + roff,
                               static_cast<const char*>(a.wu) + roff};
  f32x4v acc[2];
  acc[0] = f32x4v{0.f, 0.f, 0.f, 0.f};
  acc[1] = acc[0];
  stream_rows<WT, 2>(arow, wrow, a.H, wave, g, acc);

#pragma unroll
  for (int v = 0; v < 4; ++v) {
    red[wave][0][v][lane] = acc[0][v];
    red[wave][1][v][lane] = acc[1][v];
  }
  __syncthreads();
  if (wave != 0) return;
  // 16x16 accumulator layout: lane l holds column l%16, rows 4*(l/16) + v
  const int col = n0 + i;
  if (col >= a.F) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * g + v;
    if (row >= ne) continue;
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      gs += red[w][0][v][lane];
      us += red[w][1][v][lane];
    }
    if (WT == WT_I8) {
      gs *= a.sg[(int64_t)e * a.F + col];
      us *= a.su[(int64_t)e * a.F + col];
    }
    static_cast<uint16_t*>(a.h)[(int64_t)(r0 + row) * a.F + col] = f32_to_bf16_bits(swiglu(gs, us));
  }
}

// Kernel 2: y = h W_down^T for <= 16 rows per expert.
template <int WT>
__global__ __launch_bounds__(kWaves * 64) void down_decode_kernel(FfnArgs a) {
  __shared__ float red[kWaves][4][64];
  const int nt_per_e = (a.H + 15) / 16;
  const int e = blockIdx.x / nt_per_e;
  const int n0 = (blockIdx.x % nt_per_e) * 16;
  const int r0 = a.offsets[e];
  const int ne = a.offsets[e + 1] - r0;
  if (ne <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const uint16_t* arow = i < ne ? static_cast<const uint16_t*>(a.h) + (int64_t)(r0 + i) * a.F
                                : nullptr;
  const int n = min(n0 + i, a.H - 1);
  constexpr int ESZ = WT == WT_I8 ? 1 : 2;
  const char* const wrow[1] = {static_cast<const char*>(a.wd) +
                               ((int64_t)e * a.H + n) * a.F * ESZ};
  f32x4v acc[1];
  acc[0] = f32x4v{0.f, 0.f, 0.f, 0.f};
  stream_rows<WT, 1>(arow, wrow, a.F, wave, g, acc);

#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][v][lane] = acc[0][v];
  __syncthreads();
  if (wave != 0) return;
  const int col = n0 + i;
  if (col >= a.H) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * g + v;
    if (row >= ne) continue;
    float ys = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ys += red[w][v][lane];
    if (WT == WT_I8) ys *= a.sd[(int64_t)e * a.H + col];
    static_cast<uint16_t*>(a.y)[(int64_t)(r0 + row) * a.H + col] = f32_to_bf16_bits(ys);
  }
}

}  // namespace

hipError_t launch_gateup_decode(const FfnArgs& a, Wt wt, hipStream_t s) {
  const dim3 grid((unsigned)(a.E * ((a.F + 15) / 16)));
  if (wt == WT_I8)
    hipLaunchKernelGGL(gateup_decode_kernel<WT_I8>, grid, dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(gateup_decode_kernel<WT_BF16>, grid, dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_decode(const FfnArgs& a, Wt wt, hipStream_t s) {
  const dim3 grid((unsigned)(a.E * ((a.H + 15) / 16)));
  if (wt == WT_I8)
    hipLaunchKernelGGL(down_decode_kernel<WT_I8>, grid, dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(down_decode_kernel<WT_BF16>, grid, dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
