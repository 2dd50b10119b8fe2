// The layer's backward: everything around the GEMMs (those are in ffn_tiled.hip).
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?": the layer
// of section "The high-level architecture" (router, top-2 softmax over the
// selected logits, SwiGLU experts of section "Expert implementation: SwiGLU
// at scale", weighted combine) with the capacity drop of section "Routing:
// top-2 without auxiliary loss", which the page applies in training. The
// page gives only the forward; these kernels are its chain rule:
//
//   combine_bwd:  dw[t,j] = dout_t . y_r, dy_r = w[t,j] dout_t (kept slot
//                 (t,j) in dispatch row r), and the softmax over the selected
//                 logits: dl[t, idx[t,j]] = w_j (dw_j - sum_j' w_j' dw_j').
//   swiglu_bwd:   dg = dh u silu'(g), du = dh silu(g), stored side by side
//                 as one row [dg | du] of 2F.
//   dx_combine:   dx_t = sum over kept slots of dx_r + sum_j dl[t,idx_j] Wr[idx_j].
//   router wgrad: dWr[e] = sum_t dl[t,e] x_t.
// Every reduction runs in a fixed order (no atomics): results are
// deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

MOE_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
MOE_DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// One wave per token: dw, dy and the selected-logit gradient.
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y,
    const int32_t* __restrict__ slot_row, const float* __restrict__ w,
    const int32_t* __restrict__ idx, int64_t T, int H, int E, int k,
    uint16_t* __restrict__ dy, float* __restrict__ dw, float* __restrict__ dl) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  int r[4];
  float wt[4], dot[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = j < k ? slot_row[t * k + j] : -1;
    wt[j] = j < k ? w[t * k + j] : 0.f;
    dot[j] = 0.f;
  }
  const uint16_t* drow = dout + t * H;
  for (int c = lane; c < H / 8; c += 64) {
    const u32x4 d = ld16(drow + c * 8);
    float df[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      df[2 * q] = bf16lo(d[q]);
      df[2 * q + 1] = bf16hi(d[q]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (r[j] < 0) continue;
      const u32x4 yv = ld16(y + (int64_t)r[j] * H + c * 8);
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dot[j] += df[2 * q] * bf16lo(yv[q]);
        dot[j] += df[2 * q + 1] * bf16hi(yv[q]);
        o[q] = pack_bf16x2(wt[j] * df[2 * q], wt[j] * df[2 * q + 1]);
      }
      st16(dy + (int64_t)r[j] * H + c * 8, u32x4{o[0], o[1], o[2], o[3]});
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    dot[j] = r[j] >= 0 ? wave_sum_xor(dot[j]) : 0.f;   // r[j] is uniform over the wave
    s += wt[j] * dot[j];
  }
  if (lane < k) {
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) v = j == lane ? dot[j] : v;
    dw[t * k + lane] = v;
  }
  if (lane < E) {
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < k && idx[t * k + j] == lane) v = wt[j] * (dot[j] - s);
    dl[t * E + lane] = v;
  }
}

// dg = dh u silu'(g), du = dh silu(g) for the kept rows, 8 columns per lane.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(
    const uint16_t* __restrict__ dh, const uint16_t* __restrict__ g,
    const uint16_t* __restrict__ u, const int32_t* __restrict__ offsets, int E, int F,
    uint16_t* __restrict__ dgu) {
  const int64_t n = offsets[E];
  const int cpr = F / 8;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n * cpr;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = q / cpr;
    const int c = (int)(q - r * cpr);
    const int64_t o = r * F + c * 8;
    const u32x4 vd = ld16(dh + o), vg = ld16(g + o), vu = ld16(u + o);
    uint32_t og[4], ou[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float rg[2], ru[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float d = h ? bf16hi(vd[i]) : bf16lo(vd[i]);
        const float gg = h ? bf16hi(vg[i]) : bf16lo(vg[i]);
        const float uu = h ? bf16hi(vu[i]) : bf16lo(vu[i]);
        const float sg = 1.0f / (1.0f + __expf(-gg));
        rg[h] = d * uu * (sg + gg * sg * (1.0f - sg));
        ru[h] = d * (gg * sg);
      }
      og[i] = pack_bf16x2(rg[0], rg[1]);
      ou[i] = pack_bf16x2(ru[0], ru[1]);
    }
    st16(dgu + r * 2 * F + c * 8, u32x4{og[0], og[1], og[2], og[3]});
    st16(dgu + r * 2 * F + F + c * 8, u32x4{ou[0], ou[1], ou[2], ou[3]});
  }
}

// One wave per token: slots in order j = 0.., then the router terms in the
// same slot order, summed in float32 and rounded once.
__global__ __launch_bounds__(256) void dx_combine_kernel(
    const uint16_t* __restrict__ dxr, const int32_t* __restrict__ slot_row,
    const int32_t* __restrict__ idx, const float* __restrict__ dl, const float* __restrict__ wr,
    int64_t T, int H, int E, int k, uint16_t* __restrict__ dx) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  int r[4], ex[4];
  float gl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = j < k ? slot_row[t * k + j] : -1;
    ex[j] = j < k ? idx[t * k + j] : 0;
    gl[j] = j < k ? dl[t * E + ex[j]] : 0.f;
  }
  for (int c = lane; c < H / 8; c += 64) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (r[j] < 0) continue;
      const u32x4 v = ld16(dxr + (int64_t)r[j] * H + c * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16lo(v[q]);
        acc[2 * q + 1] += bf16hi(v[q]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= k) continue;
      const float* wrow = wr + (int64_t)ex[j] * H + c * 8;
      const f32x4 a = *reinterpret_cast<const f32x4*>(wrow);
      const f32x4 b = *reinterpret_cast<const f32x4*>(wrow + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += gl[j] * a[i];
        acc[4 + i] += gl[j] * b[i];
      }
    }
    st16(dx + t * H + c * 8, u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])});
  }
}

// Router weight gradient, pass 1: part[c][e][h] = sum over the tokens of
// chunk c (ascending) of dl[t,e] x[t,h]; 2 columns per thread. Pass 2 sums
// the chunks in order. Chunks hold 128 tokens, or more when T > 2^22 so
// that there are at most 32768 of them.
int64_t router_chunk_len(int64_t T) { return T <= (128ll << 15) ? 128 : (T + 32767) / 32768; }

__global__ __launch_bounds__(256) void router_wgrad_part_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dl, int64_t T, int H, int E,
    int64_t chunk, float* __restrict__ part) {
  const int h = (blockIdx.x * 256 + threadIdx.x) * 2;
  const int64_t t0 = (int64_t)blockIdx.y * chunk;
  const int64_t t1 = min(t0 + chunk, T);
  if (h >= H) return;
  float acc[16][2];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e][0] = acc[e][1] = 0.f;
  for (int64_t t = t0; t < t1; ++t) {
    const uint32_t xv = *reinterpret_cast<const uint32_t*>(x + t * H + h);
    const float x0 = bf16lo(xv), x1 = bf16hi(xv);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (e >= E) break;
      const float d = dl[t * E + e];
      acc[e][0] += d * x0;
      acc[e][1] += d * x1;
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (e >= E) break;
    float* p = part + ((int64_t)blockIdx.y * E + e) * H + h;
    p[0] = acc[e][0];
    p[1] = acc[e][1];
  }
}

__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(const float* __restrict__ part,
                                                                  int nchunk, int H, int E,
                                                                  float* __restrict__ dwr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)E * H) return;
  float s = 0.f;
  for (int c = 0; c < nchunk; ++c) s += part[(int64_t)c * E * H + i];
  dwr[i] = s;
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

unsigned stride_grid(int64_t items) {
  const int64_t g = (items + 255) / 256;
  return (unsigned)(g < 1 ? 1 : g > 65536 ? 65536 : g);
}

}  // namespace

int64_t router_wgrad_chunks(int64_t T) {
  const int64_t c = router_chunk_len(T);
  return (T + c - 1) / c;
}

hipError_t launch_combine_bwd(const void* dout, const void* y, const int32_t* slot_row,
                              const float* w, const int32_t* idx, int64_t T, int H, int E, int k,
                              void* dy, float* dw, float* dl, hipStream_t s) {
  hipLaunchKernelGGL(combine_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(y), slot_row,
                     w, idx, T, H, E, k, static_cast<uint16_t*>(dy), dw, dl);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* dh, const void* g, const void* u, const int32_t* offsets,
                             int E, int64_t max_rows, int F, void* dgu, hipStream_t s) {
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(stride_grid(max_rows * (F / 8))), dim3(256), 0, s,
                     static_cast<const uint16_t*>(dh), static_cast<const uint16_t*>(g),
                     static_cast<const uint16_t*>(u), offsets, E, F, static_cast<uint16_t*>(dgu));
  return hipGetLastError();
}

hipError_t launch_dx_combine(const void* dxr, const int32_t* slot_row, const int32_t* idx,
                             const float* dl, const float* wr, int64_t T, int H, int E, int k,
                             void* dx, hipStream_t s) {
  hipLaunchKernelGGL(dx_combine_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(dxr), slot_row, idx, dl, wr, T, H, E, k,
                     static_cast<uint16_t*>(dx));
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const void* x, const float* dl, int64_t T, int H, int E,
                               float* part, float* dwr, hipStream_t s) {
  const int64_t nchunk = router_wgrad_chunks(T);
  if (nchunk == 0) {
    hipLaunchKernelGGL(fill_f32_kernel, dim3(stride_grid((int64_t)E * H)), dim3(256), 0, s, dwr,
                       (int64_t)E * H, 0.f);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(router_wgrad_part_kernel, dim3((unsigned)((H / 2 + 255) / 256), (unsigned)nchunk),
                     dim3(256), 0, s, static_cast<const uint16_t*>(x), dl, T, H, E,
                     router_chunk_len(T), part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(router_wgrad_reduce_kernel, dim3((unsigned)(((int64_t)E * H + 255) / 256)),
                     dim3(256), 0, s, part, (int)nchunk, H, E, dwr);
  return hipGetLastError();
}

}  // namespace moe
