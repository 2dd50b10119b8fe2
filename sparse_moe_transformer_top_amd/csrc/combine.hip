// Weighted combine of each token's expert outputs back to token order.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?":
// GrokMoELayer.forward ends with dispatch-and-combine, and the expert-parallel
// pseudocode (section "Expert parallelism vs. tensor parallelism") scales each
// expert's output by the token's routing weight for that expert.
//
// Gather form: each thread owns 8 consecutive hidden elements of one token and
// reads the token's kept expert rows through slot_row, summing in float32 in
// slot order; one rounding to the output dtype at the end. No atomics, so the
// result is deterministic. HBM-bound: reads k rows of y_perm, writes one row.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <int ACT>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const void* __restrict__ yv, const int32_t* __restrict__ slot_row,
    const float* __restrict__ w, int64_t T, int H, int k, void* __restrict__ outv) {
  const int chunks = H / 8;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= T * chunks) return;
  const int64_t t = gid / chunks;
  const int c = (int)(gid - t * chunks);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int32_t r = slot_row[t * k + j];
    if (r < 0) continue;
    const float wj = w[t * k + j];
    if (ACT == ACT_BF16) {
      const uint4 v = *reinterpret_cast<const uint4*>(
          static_cast<const uint16_t*>(yv) + (int64_t)r * H + c * 8);
      acc[0] = fmaf(wj, bf16lo(v.x), acc[0]); acc[1] = fmaf(wj, bf16hi(v.x), acc[1]);
      acc[2] = fmaf(wj, bf16lo(v.y), acc[2]); acc[3] = fmaf(wj, bf16hi(v.y), acc[3]);
      acc[4] = fmaf(wj, bf16lo(v.z), acc[4]); acc[5] = fmaf(wj, bf16hi(v.z), acc[5]);
      acc[6] = fmaf(wj, bf16lo(v.w), acc[6]); acc[7] = fmaf(wj, bf16hi(v.w), acc[7]);
    } else {
      const float4* p = reinterpret_cast<const float4*>(
          static_cast<const float*>(yv) + (int64_t)r * H + c * 8);
      const float4 a = p[0], b = p[1];
      acc[0] = fmaf(wj, a.x, acc[0]); acc[1] = fmaf(wj, a.y, acc[1]);
      acc[2] = fmaf(wj, a.z, acc[2]); acc[3] = fmaf(wj, a.w, acc[3]);
      acc[4] = fmaf(wj, b.x, acc[4]); acc[5] = fmaf(wj, b.y, acc[5]);
      acc[6] = fmaf(wj, b.z, acc[6]); acc[7] = fmaf(wj, b.w, acc[7]);
    }
  }
  if (ACT == ACT_BF16) {
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(outv) + t * H + c * 8) = o;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(outv) + t * H + c * 8);
    p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

}  // namespace

hipError_t launch_combine(const void* y_perm, const int32_t* slot_row, const float* w, int64_t T,
                          int H, int k, Act act, void* out, hipStream_t s) {
  const int64_t items = T * (H / 8);
  const dim3 grid((unsigned)((items + kThreads - 1) / kThreads));
  if (act == ACT_BF16)
    hipLaunchKernelGGL(combine_kernel<ACT_BF16>, grid, dim3(kThreads), 0, s, y_perm, slot_row, w,
                       T, H, k, out);
  else
    hipLaunchKernelGGL(combine_kernel<ACT_F32>, grid, dim3(kThreads), 0, s, y_perm, slot_row, w,
                       T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
