// Routing statistics from the router's logits and the dispatch counts.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section
// "Routing: top-2 without auxiliary loss": after training the page counts
// each expert's share of the top-2 picks (utilisation, 1.0 per expert for a
// balanced router) and notes that the top-2 logits usually stand clear of the
// 3rd expert while the 3rd and 4th keep noticeable probability. Per token
// this kernel gives the margin l_(k) - l_(k+1) and the full-softmax mass
// outside the selected k; per expert, counts * E / (T*k).
//
// One thread per token (E <= 16 logits in registers): the k largest are taken
// one at a time as in the router (larger value first, lower index among equal
// values), then the best remaining one; the softmax uses the row maximum.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <int EC>
__global__ __launch_bounds__(256) void routing_stats_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ counts, int64_t T, int E, int k,
    float* __restrict__ util, float* __restrict__ margin, float* __restrict__ mass) {
  if (util && blockIdx.x == 0 && (int)threadIdx.x < E)
    util[threadIdx.x] =
        T > 0 ? (float)((double)counts[threadIdx.x] * E / ((double)T * k)) : 0.f;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T || !(margin || mass)) return;
  float l[EC];
#pragma unroll
  for (int e = 0; e < EC; ++e) l[e] = e < E ? logits[t * E + e] : 0.f;
  uint32_t taken = 0;
  float last = 0.f;
  for (int j = 0; j < k; ++j) {
    int bi = -1;
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (e < E && !((taken >> e) & 1u) && (bi < 0 || l[e] > l[bi])) bi = e;
    taken |= 1u << bi;
    last = l[bi];
  }
  if (margin) {
    float next = 0.f;
    bool any = false;
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (e < E && !((taken >> e) & 1u) && (!any || l[e] > next)) {
        next = l[e];
        any = true;
      }
    margin[t] = any ? last - next : INFINITY;
  }
  if (mass) {
    float mx = l[0];
#pragma unroll
    for (int e = 1; e < EC; ++e)
      if (e < E) mx = fmaxf(mx, l[e]);
    float zs = 0.f, zo = 0.f;
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      if (e < E) {
        const float z = expf(l[e] - mx);
        zs += z;
        if (!((taken >> e) & 1u)) zo += z;
      }
    }
    mass[t] = zo / zs;
  }
}

}  // namespace

hipError_t launch_routing_stats(const float* logits, const int32_t* counts, int64_t T, int E,
                                int k, float* util, float* margin, float* mass, hipStream_t s) {
  const dim3 grid((unsigned)(T > 0 ? (T + 255) / 256 : 1));
  if (E <= 8)
    hipLaunchKernelGGL(routing_stats_kernel<8>, grid, dim3(256), 0, s, logits, counts, T, E, k,
                       util, margin, mass);
  else
    hipLaunchKernelGGL(routing_stats_kernel<16>, grid, dim3(256), 0, s, logits, counts, T, E, k,
                       util, margin, mass);
  return hipGetLastError();
}

}  // namespace moe
