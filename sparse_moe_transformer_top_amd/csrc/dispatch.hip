// Dispatch: group the token->expert assignments by expert in token order and
// drop the assignments over capacity.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section
// "Routing: top-2 without auxiliary loss": grok_router_forward builds a one-hot
// dispatch mask from the top-k indices and, with a finite capacity factor,
// drops what overflows an expert's capacity (factor 1.25 in training, no drop
// at inference). Here the mask is kept in index form: per-expert counts and
// offsets, the row permutation and each assignment's row.
//
// Rule: an assignment's rank in its expert is the number of earlier tokens
// that chose the same expert; it is kept iff rank < cap. Ranks come from wave
// ballots and per-wave counts scanned in wave order, so they are exact and
// deterministic (no atomic slot claiming).
//
// Two kernels, 1024 tokens per work-group: (1) per-block expert histogram;
// (2) every block derives its starting rank per expert from the histograms of
// the blocks before it, ranks its tokens and scatters. Up to 1024 tokens the
// first kernel is skipped.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBlockTokens = 1024;
constexpr int kMaxE = 16;
constexpr int kWavesPerBlock = kBlockTokens / 64;

__global__ __launch_bounds__(kBlockTokens) void dispatch_hist_kernel(
    const int32_t* __restrict__ idx, int64_t T, int E, int k, int32_t* __restrict__ hist) {
  __shared__ int32_t s_hist[kMaxE];
  if (threadIdx.x < kMaxE) s_hist[threadIdx.x] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kBlockTokens + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) atomicAdd(&s_hist[e], 1);  // integer adds: order-free
    }
  }
  __syncthreads();
  if (threadIdx.x < E) hist[(int64_t)blockIdx.x * E + threadIdx.x] = s_hist[threadIdx.x];
}

// With nblk == 1 (all tokens in this block) the histogram pass is skipped and
// the block's own ballot counts are the totals.
__global__ __launch_bounds__(kBlockTokens) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int E, int k, int64_t cap, int nblk,
    const int32_t* __restrict__ hist, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ slot_row, uint8_t* __restrict__ dropped) {
  __shared__ int32_t s_base[kMaxE];                 // rank of this block's first token per expert
  __shared__ int32_t s_total[kMaxE];                // assignments per expert over all blocks
  __shared__ int32_t s_off[kMaxE + 1];              // row offsets per expert
  __shared__ int32_t s_wcnt[kMaxE][kWavesPerBlock];  // per-wave counts -> exclusive wave bases
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int blk = blockIdx.x;

  const int64_t t = (int64_t)blk * kBlockTokens + tid;
  const bool valid = t < T;
  int ej[4] = {-1, -1, -1, -1};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < k && valid) {
      const int e = idx[t * k + j];
      ej[j] = (e >= 0 && e < E) ? e : -1;   // an out-of-range id is treated as dropped
    }
  }

  // in-block stable ranks: ballot per expert, popcount of the lower lanes
  const uint64_t lt_mask = lane ? (~0ull >> (64 - lane)) : 0ull;
  int lrank[4] = {0, 0, 0, 0};
  for (int e = 0; e < E; ++e) {
    bool pred = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) pred |= (j < k) && ej[j] == e;
    const uint64_t m = __ballot(pred);
    const int r = __popcll(m & lt_mask);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < k && ej[j] == e) lrank[j] = r;
    if (lane == 0) s_wcnt[e][wave] = __popcll(m);
  }
  __syncthreads();
  if (tid < E) {
    int32_t run = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      const int32_t c = s_wcnt[tid][w];
      s_wcnt[tid][w] = run;
      run += c;
    }
    int32_t base = 0, total = run;
    if (nblk > 1) {
      total = 0;
      for (int b = 0; b < nblk; ++b) {
        const int32_t c = hist[(int64_t)b * E + tid];
        if (b < blk) base += c;
        total += c;
      }
    }
    s_base[tid] = base;
    s_total[tid] = total;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t run = 0;
    for (int e = 0; e < E; ++e) {
      const int32_t total = s_total[e];
      const int32_t kept = (cap >= 0 && total > cap) ? (int32_t)cap : total;
      s_off[e] = run;
      if (blk == 0) { counts[e] = total; offsets[e] = run; }
      run += kept;
    }
    s_off[E] = run;
    if (blk == 0) offsets[E] = run;
  }
  __syncthreads();

  if (valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= k) break;
      const int e = ej[j];
      const int64_t a = t * k + j;
      const int32_t rank = e >= 0 ? s_base[e] + s_wcnt[e][wave] + lrank[j] : 0;
      if (e >= 0 && (cap < 0 || rank < cap)) {
        const int32_t row = s_off[e] + rank;
        perm[row] = (int32_t)a;
        slot_row[a] = row;
        dropped[a] = 0;
      } else {
        slot_row[a] = -1;
        dropped[a] = 1;
      }
    }
  }
  // rows past the kept total hold -1
  const int64_t n_kept = s_off[E];
  const int64_t a0 = (int64_t)blk * kBlockTokens * k;
  const int64_t a1 = min(a0 + (int64_t)kBlockTokens * k, T * k);
  for (int64_t a = a0 + tid; a < a1; a += kBlockTokens)
    if (a >= n_kept) perm[a] = -1;
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

size_t dispatch_ws_bytes(int64_t T, int E) {
  const int64_t nblk = (T + kBlockTokens - 1) / kBlockTokens;
  return (size_t)(nblk > 0 ? nblk : 1) * E * sizeof(int32_t);
}

hipError_t launch_dispatch(const int32_t* idx, int64_t T, int E, int k, int64_t cap,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_row,
                           uint8_t* dropped, void* ws, hipStream_t s) {
  const int nblk = (int)((T + kBlockTokens - 1) / kBlockTokens);
  int32_t* hist = static_cast<int32_t*>(ws);
  if (nblk > 1) {
    hipLaunchKernelGGL(dispatch_hist_kernel, dim3(nblk), dim3(kBlockTokens), 0, s, idx, T, E, k,
                       hist);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(nblk), dim3(kBlockTokens), 0, s, idx, T, E, k,
                     cap, nblk, hist, counts, offsets, perm, slot_row, dropped);
  return hipGetLastError();
}

}  // namespace moe
