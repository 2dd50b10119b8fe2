// Router linear + top-k + softmax over the selected logits, one fused kernel.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?": the router
// is a bias-free linear from the hidden size to the expert logits, followed by
// torch.topk (largest first) and a softmax over only the k selected values
// (section "Routing: top-2 without auxiliary loss", grok_router_forward;
// section "The high-level architecture", GrokMoELayer.forward).
//
// Mapping: a work-group owns kTokPerBlock tokens and its 4 waves split the
// hidden dimension into 4 contiguous quarters, so that a decode batch of a few
// tokens still runs 4 short dependency chains per token group instead of one
// long one. Lanes split a wave's quarter into 8-element chunks (16-byte loads
// of bf16 x, 32 bytes of the float32 router row per expert); each router
// chunk is loaded once and reused for all the block's tokens. Partial dot
// products are reduced across the block's 256 lanes through LDS in a fixed
// order, so logits are deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 4;
constexpr int kWaves = 4;

template <int ACT>
MOE_DEV void load_x8(const void* xv, int64_t t, int H, int h0, float (&xo)[8]) {
  if (ACT == ACT_BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(xv) + t * H + h0);
    xo[0] = bf16lo(v.x); xo[1] = bf16hi(v.x); xo[2] = bf16lo(v.y); xo[3] = bf16hi(v.y);
    xo[4] = bf16lo(v.z); xo[5] = bf16hi(v.z); xo[6] = bf16lo(v.w); xo[7] = bf16hi(v.w);
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(xv) + t * H + h0);
    const float4 a = p[0], b = p[1];
    xo[0] = a.x; xo[1] = a.y; xo[2] = a.z; xo[3] = a.w;
    xo[4] = b.x; xo[5] = b.y; xo[6] = b.z; xo[7] = b.w;
  }
}

// Select the k largest of l[0..E) (descending; equal values: lower index
// first) and write indices, softmax weights and optionally the logits.
template <int EC>
MOE_DEV void select_topk(const float (&l)[EC], int E, int k, int64_t t, int32_t* idx,
                         float* w, float* logits) {
  uint32_t taken = 0;
  int si[4] = {0, 0, 0, 0};
  float sv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < k) {
      float best = 0.f;
      int bi = -1;
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        const bool ok = e < E && !((taken >> e) & 1u);
        if (ok && (bi < 0 || l[e] > best)) { best = l[e]; bi = e; }
      }
      taken |= 1u << bi;
      si[j] = bi;
      sv[j] = best;
    }
  }
  float z[4], zs = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    z[j] = j < k ? expf(sv[j] - sv[0]) : 0.f;
    zs += z[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < k) {
      idx[t * k + j] = si[j];
      w[t * k + j] = z[j] / zs;
    }
  }
  if (logits) {
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (e < E) logits[t * E + e] = l[e];
  }
}

// Cross-lane reduction through LDS: every lane stores its kTokPerBlock*EC
// partial sums as one 256-value row per (token, expert), in 8 segments of 32
// (one pad float per segment so that the 64 lanes of the second pass, which
// read 8 rows x 8 segments, hit 64 distinct banks). Pass 2 sums each segment
// in lane order, pass 3 the 8 segment sums: a fixed order, so logits are
// deterministic, and little code (the kernel runs once per wave at decode
// sizes, where instruction fetch dominates).
constexpr int kLanes = kWaves * 64;          // 256 partial sums per (token, expert)
constexpr int kSeg = 8, kSegLen = kLanes / kSeg, kSegStride = kSegLen + 1;
constexpr int kRowStride = kSeg * kSegStride;

template <int EC, int ACT>
__global__ __launch_bounds__(kWaves * 64) void router_topk_kernel(
    const void* __restrict__ x, const float* __restrict__ wr, int64_t T, int H, int E, int k,
    int32_t* __restrict__ idx, float* __restrict__ w, float* __restrict__ logits) {
  constexpr int NV = kTokPerBlock * EC;
  __shared__ float red[NV * kRowStride];
  __shared__ float seg[NV][kSeg];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerBlock;

  float acc[kTokPerBlock][EC];
#pragma unroll
  for (int i = 0; i < kTokPerBlock; ++i)
#pragma unroll
    for (int e = 0; e < EC; ++e) acc[i][e] = 0.f;

  // this wave's quarter of the hidden dimension, in 8-element chunks. The
  // loads of a chunk carry no conditions (token and expert indices are
  // clamped; results for tokens past T and experts past E are never used).
  const int chunks = H / 8;
  const int c_begin = (chunks * wave) / kWaves, c_end = (chunks * (wave + 1)) / kWaves;
  int64_t trow[kTokPerBlock];
#pragma unroll
  for (int tt = 0; tt < kTokPerBlock; ++tt) trow[tt] = min(t0 + tt, T - 1);
  for (int c = c_begin + lane; c < c_end; c += 64) {
    const int h0 = c * 8;
    float xv[kTokPerBlock][8];
#pragma unroll
    for (int tt = 0; tt < kTokPerBlock; ++tt) load_x8<ACT>(x, trow[tt], H, h0, xv[tt]);
#pragma unroll
    for (int e0 = 0; e0 < EC; e0 += 8) {
      float wv[8][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4* p = reinterpret_cast<const float4*>(wr + (int64_t)min(e0 + e, E - 1) * H + h0);
        const float4 a = p[0], b = p[1];
        wv[e][0] = a.x; wv[e][1] = a.y; wv[e][2] = a.z; wv[e][3] = a.w;
        wv[e][4] = b.x; wv[e][5] = b.y; wv[e][6] = b.z; wv[e][7] = b.w;
      }
#pragma unroll
      for (int tt = 0; tt < kTokPerBlock; ++tt)
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            acc[tt][e0 + e] = fmaf(xv[tt][i], wv[e][i], acc[tt][e0 + e]);
    }
  }

  // pass 1: lane tid's partial sums go to position tid of every row
  const int pos = (tid / kSegLen) * kSegStride + tid % kSegLen;
#pragma unroll
  for (int tt = 0; tt < kTokPerBlock; ++tt)
#pragma unroll
    for (int e = 0; e < EC; ++e) red[(tt * EC + e) * kRowStride + pos] = acc[tt][e];
  __syncthreads();
  // pass 2: segment sums, in lane order
  for (int j = tid; j < NV * kSeg; j += kLanes) {
    const float* r = red + (j / kSeg) * kRowStride + (j % kSeg) * kSegStride;
    float v = 0.f;
#pragma unroll 8
    for (int i = 0; i < kSegLen; ++i) v += r[i];
    seg[j / kSeg][j % kSeg] = v;
  }
  __syncthreads();
  // pass 3: one lane per token adds its segment sums and selects
  if (tid < kTokPerBlock && t0 + tid < T) {
    float l[EC];
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < kSeg; ++q) v += seg[tid * EC + e][q];
      l[e] = v;
    }
    select_topk<EC>(l, E, k, t0 + tid, idx, w, logits);
  }
}

template <int EC>
hipError_t launch_ec(const void* x, Act act, const float* wr, int64_t T, int H, int E, int k,
                     int32_t* idx, float* w, float* logits, hipStream_t s) {
  const dim3 grid((unsigned)((T + kTokPerBlock - 1) / kTokPerBlock));
  if (act == ACT_BF16)
    hipLaunchKernelGGL((router_topk_kernel<EC, ACT_BF16>), grid, dim3(kWaves * 64), 0, s, x, wr,
                       T, H, E, k, idx, w, logits);
  else
    hipLaunchKernelGGL((router_topk_kernel<EC, ACT_F32>), grid, dim3(kWaves * 64), 0, s, x, wr,
                       T, H, E, k, idx, w, logits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_topk(const void* x, Act act, const float* wr, int64_t T, int H, int E,
                              int k, int32_t* idx, float* w, float* logits, hipStream_t s) {
  if (E <= 8) return launch_ec<8>(x, act, wr, T, H, E, k, idx, w, logits, s);
  return launch_ec<16>(x, act, wr, T, H, E, k, idx, w, logits, s);
}

}  // namespace moe
