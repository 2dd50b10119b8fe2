// Expert-parallel layouts on either side of the all-to-all.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section
// "Expert parallelism vs. tensor parallelism": with experts placed on ranks,
// each rank routes its own tokens, sends every token to the ranks of its
// experts, runs its local experts and gathers the outputs back (the EP
// forward pseudocode). Experts sit in contiguous blocks: rank r holds experts
// r*E/R ... (r+1)*E/R - 1, so the dispatch order (rows grouped by expert) is
// already grouped by destination rank.
//
//   pack:        send[j] = x[perm[j] / k] for the kept rows j < offsets[E];
//                rows per destination rank from the offsets.
//   recv layout: the receive buffer holds each source rank's rows grouped by
//                local expert; the grouped GEMM wants them grouped by local
//                expert, then source. Instead of moving rows, this computes
//                the expert offsets and, for each row in that order, its
//                position in the receive buffer: the GEMM gathers through
//                that index (perm with k = 1).
//   unpack:      back[row_index[j]] = y[j]: expert outputs in receive order
//                for the return exchange, after which each source holds its
//                rows in its own dispatch order, ready for moe_combine.
// Rows move as 16-byte chunks; everything is index arithmetic, no floats.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

MOE_DEV u32x4 ld16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

__global__ __launch_bounds__(256) void ep_pack_kernel(const char* __restrict__ x,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      int k, int R, int64_t row_bytes,
                                                      char* __restrict__ send,
                                                      int32_t* __restrict__ send_counts) {
  if (blockIdx.x == 0 && (int)threadIdx.x < R) {
    const int per = E / R;
    send_counts[threadIdx.x] = offsets[(threadIdx.x + 1) * per] - offsets[threadIdx.x * per];
  }
  const int64_t n = offsets[E];
  const int64_t chunks = row_bytes / 16;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n * chunks;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = q / chunks, c = q - row * chunks;
    const int64_t tok = perm[row] / k;
    *reinterpret_cast<u32x4*>(send + row * row_bytes + c * 16) =
        ld16(x + tok * row_bytes + c * 16);
  }
}

// One work-group per (local expert e, source p) segment; segment starts are
// prefix sums over the small R x E_local count matrix. Rows whose regrouped
// position reaches max_rows are not written; the offsets are capped there.
__global__ __launch_bounds__(256) void ep_recv_layout_kernel(const int32_t* __restrict__ counts,
                                                             int R, int El, int64_t max_rows,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ row_index) {
  const int e = blockIdx.x / R, p = blockIdx.x % R;
  __shared__ int64_t s_in, s_out;
  if (threadIdx.x == 0) {
    int64_t in = 0, out = 0;   // position in the receive buffer / in the regrouped order
    for (int q = 0; q < p * El + e; ++q) in += counts[q];
    for (int ee = 0; ee < e; ++ee)
      for (int pp = 0; pp < R; ++pp) out += counts[pp * El + ee];
    for (int pp = 0; pp < p; ++pp) out += counts[pp * El + e];
    s_in = in;
    s_out = out;
  }
  if (blockIdx.x == 0 && (int)threadIdx.x <= El) {
    int64_t o = 0;
    for (int ee = 0; ee < (int)threadIdx.x; ++ee)
      for (int pp = 0; pp < R; ++pp) o += counts[pp * El + ee];
    offsets[threadIdx.x] = (int32_t)min(o, max_rows);
  }
  __syncthreads();
  const int64_t c = counts[p * El + e];
  for (int64_t t = threadIdx.x; t < c; t += blockDim.x) {
    const int64_t o = s_out + t;
    if (o < max_rows) row_index[o] = (int32_t)(s_in + t);
  }
}

__global__ __launch_bounds__(256) void ep_unpack_kernel(const char* __restrict__ y,
                                                        const int32_t* __restrict__ row_index,
                                                        const int32_t* __restrict__ offsets,
                                                        int El, int64_t row_bytes,
                                                        char* __restrict__ back) {
  const int64_t n = offsets[El];
  const int64_t chunks = row_bytes / 16;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n * chunks;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = q / chunks, c = q - j * chunks;
    *reinterpret_cast<u32x4*>(back + (int64_t)row_index[j] * row_bytes + c * 16) =
        ld16(y + j * row_bytes + c * 16);
  }
}

unsigned stride_grid(int64_t items) {
  const int64_t g = (items + 255) / 256;
  return (unsigned)(g < 1 ? 1 : g > 16384 ? 16384 : g);
}

}  // namespace

hipError_t launch_ep_pack(const void* x, int64_t row_bytes, const int32_t* perm,
                          const int32_t* offsets, int64_t max_rows, int E, int k, int R,
                          void* send, int32_t* send_counts, hipStream_t s) {
  hipLaunchKernelGGL(ep_pack_kernel, dim3(stride_grid(max_rows * (row_bytes / 16))), dim3(256), 0,
                     s, static_cast<const char*>(x), perm, offsets, E, k, R, row_bytes,
                     static_cast<char*>(send), send_counts);
  return hipGetLastError();
}

hipError_t launch_ep_recv_layout(const int32_t* counts, int R, int El, int64_t max_rows,
                                 int32_t* offsets, int32_t* row_index, hipStream_t s) {
  hipLaunchKernelGGL(ep_recv_layout_kernel, dim3((unsigned)(R * El)), dim3(256), 0, s, counts, R,
                     El, max_rows, offsets, row_index);
  return hipGetLastError();
}

hipError_t launch_ep_unpack(const void* y, int64_t row_bytes, const int32_t* row_index,
                            const int32_t* offsets, int El, int64_t max_rows, void* back,
                            hipStream_t s) {
  hipLaunchKernelGGL(ep_unpack_kernel, dim3(stride_grid(max_rows * (row_bytes / 16))), dim3(256),
                     0, s, static_cast<const char*>(y), row_index, offsets, El, row_bytes,
                     static_cast<char*>(back));
  return hipGetLastError();
}

}  // namespace moe
