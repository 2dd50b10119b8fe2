// Router linear + top-k + softmax over the selected logits, one fused kernel.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?": the router
// is a bias-free linear from the hidden size to the expert logits, followed by
// torch.topk (largest first) and a softmax over only the k selected values
// (section "Routing: top-2 without auxiliary loss", grok_router_forward;
// section "The high-level architecture", GrokMoELayer.forward).
//
// Two kernels. For a few tokens (decode), router_topk_kernel: a work-group
// owns kTokPerBlock tokens and its 4 waves split the hidden dimension into 4
// contiguous quarters, so that a decode batch still runs 4 short dependency
// chains per token group instead of one long one. Lanes split a wave's quarter
// into 8-element chunks (16-byte loads of bf16 x, 32 bytes of the float32
// router row per expert); each router chunk is loaded once and reused for all
// the block's tokens. Partial dot products are reduced across the block's 256
// lanes through LDS in a fixed order, so logits are deterministic.
//
// For many tokens, router_mfma_kernel: the logits are a [T,H] x [H,E] product
// whose only large dimensions are T and H, and on the vector ALU (float32 FMA,
// 8 per token and hidden element) it costs about as long as reading x from
// HBM, while the per-block router reloads of the kernel above cost L2
// bandwidth on top. On the matrix cores it is nearly free: each float32
// router weight is split exactly into three bf16 terms, w = hi + mid + lo
// (hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid, each difference exact
// in float32 and lo exact in bf16), and a 32x32x16 bf16 MFMA takes 32 tokens
// against 24 columns (hi, mid, lo of 8 experts). Every product of a bf16 x and
// a bf16 term is exact in float32, so a logit is the exact dot product up to
// float32 accumulation, as on the vector path. The kernel is then bound by
// reading x once and each work-group's copy of the router weights (from L2).
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

// ---------------------------------------------------------------------------
// MFMA router (bf16 x, E <= 8, H a multiple of 64)
// ---------------------------------------------------------------------------
// A work-group owns 32 tokens (one MFMA row tile) and its NW waves take the
// hidden dimension in chunks of 64, round-robin (wave q: chunks q, q + NW,
// ...), so neighbouring waves read neighbouring pieces of the same x rows
// (8 or 16 waves per work-group, or 6 or 8 chunks in flight, were slower).
// Per chunk a wave (1) splits the 8 x 64 router weights into hi / mid / lo
// and writes them to its own LDS buffer as 24 rows of 64 bf16 (rows s*8 + e;
// 16-byte chunks XOR-swizzled by (row / 2) % 8, so the MFMA's B-operand reads
// of 16 rows at one chunk column hit 16 distinct 16-byte bank groups), (2)
// runs 4 MFMAs (two accumulators, so consecutive MFMAs do not wait for each
// other) with the x rows as the A operand straight from registers. x and
// router loads run D chunks ahead.
// The waves' 32 x 24 partial sums then meet in LDS (over the split buffers)
// and one lane per token adds them in a fixed order (wave, then hi, mid, lo),
// so logits are deterministic.
constexpr int kMTok = 32;            // tokens per work-group
constexpr int kMChunk = 64;          // hidden elements per chunk
constexpr int kPartStride = 25;      // floats per token row of a partial tile (24 + pad)
constexpr int kRouterWaves = 4;      // waves per work-group
constexpr int kRouterDepth = 4;      // chunks in flight per wave (even: LDS buffer parity)
// Token counts from which the MFMA kernel runs. Each work-group reads its 32
// x rows and the whole router weight (E H float32, from L2), so its time has
// a floor of ~16 us at any T; the vector kernel is faster up to ~4.5k tokens
// (at 4096: 17.0 against 17.1-17.7 us; at 8192: 29.3 against 19.4-19.6).
constexpr int64_t kMfmaRouterMinTokens = 4608;

MOE_DEV int wsplit_word(int row, int chunk) { return row * 32 + ((chunk ^ ((row >> 1) & 7)) << 2); }

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, int64_t T, int H, int E, int k,
    int32_t* __restrict__ idx, float* __restrict__ w, float* __restrict__ logits) {
  static_assert(D % 2 == 0, "two LDS buffers alternate by chunk parity");
  // per wave, two buffers of 32 rows x 64 bf16 (rows 24..31 stay zero); after
  // the k loop the same memory holds the waves' partial tiles
  __shared__ __align__(16) uint32_t wsp[NW][2][32 * 32];
  static_assert(sizeof(float) * kMTok * kPartStride <= sizeof(wsp[0]), "partials fit");
  float(*part)[kMTok][kPartStride] = reinterpret_cast<float(*)[kMTok][kPartStride]>(&wsp[0][0][0]);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kMTok;
  const int nchunks = H / kMChunk;
  const int nc = nchunks > wave ? (nchunks - wave + NW - 1) / NW : 0;   // this wave's chunks

  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int b = 0; b < 2; ++b) *reinterpret_cast<u32x4*>(&wsp[wave][b][24 * 32 + lane * 4]) = zero;

  // A operand: lane -> token row lane % 32, k half lane / 32 of each 16-k step
  const int64_t trow = min(t0 + (lane & 31), T - 1);
  const uint16_t* xrow = x + trow * H + 8 * (lane >> 5);
  // router loads: lane -> expert lane / 8 (clamped; columns past E are unused),
  // 8 consecutive k at 8 (lane % 8) of the chunk
  const int ew = lane >> 3, jw = lane & 7;
  const float* wrow = wr + (int64_t)min(ew, E - 1) * H + 8 * jw;
  // B operand: lane -> column lane % 32 (s * 8 + e), k half lane / 32
  const int bn = lane & 31, bh = lane >> 5;

  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[0][i] = acc[1][i] = 0.f;

  if (nc > 0) {
    u32x4 xa[D][4];
    f32x4 wa[D][2];
    // chunks past this wave's last one reload the last (in bounds, unused)
#define MOE_ROUTER_LOAD(SLOT, C)                                                  \
  do {                                                                            \
    const int g_ = wave + NW * min((C), nc - 1);                                  \
    const uint16_t* px_ = xrow + g_ * kMChunk;                                    \
    _Pragma("unroll") for (int ks = 0; ks < 4; ++ks)                              \
      xa[SLOT][ks] = *reinterpret_cast<const u32x4*>(px_ + ks * 16);              \
    const float* pw_ = wrow + g_ * kMChunk;                                       \
    wa[SLOT][0] = *reinterpret_cast<const f32x4*>(pw_);                           \
    wa[SLOT][1] = *reinterpret_cast<const f32x4*>(pw_ + 4);                       \
  } while (0)
#pragma unroll
    for (int d = 0; d < D; ++d) MOE_ROUTER_LOAD(d, d);
    for (int c0 = 0; c0 < nc; c0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int c = c0 + d;
        uint32_t* buf = wsp[wave][d & 1];
        // (1) exact three-term split of 8 router weights, into LDS
        u32x4 hv, mv, lv;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const f32x4 src = wa[d][p >> 1];
          const float a = src[(p & 1) * 2], b = src[(p & 1) * 2 + 1];
          const uint32_t h = pack_bf16x2(a, b);
          const float ra = a - bf16lo(h), rb = b - bf16hi(h);
          const uint32_t m = pack_bf16x2(ra, rb);
          const float sa = ra - bf16lo(m), sb = rb - bf16hi(m);
          hv[p] = h;
          mv[p] = m;
          lv[p] = pack_bf16x2(sa, sb);
        }
        *reinterpret_cast<u32x4*>(buf + wsplit_word(ew, jw)) = hv;
        *reinterpret_cast<u32x4*>(buf + wsplit_word(8 + ew, jw)) = mv;
        *reinterpret_cast<u32x4*>(buf + wsplit_word(16 + ew, jw)) = lv;
        // (2) four 16-k steps; a chunk past the wave's last adds zeros
        const bool valid = c < nc;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 bv = *reinterpret_cast<const u32x4*>(buf + wsplit_word(bn, 2 * ks + bh));
          const u32x4 av = valid ? xa[d][ks] : zero;
          acc[ks & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bv),
                                                                acc[ks & 1], 0, 0, 0);
        }
        MOE_ROUTER_LOAD(d, c + D);
      }
    }
#undef MOE_ROUTER_LOAD
  }

  __syncthreads();   // every wave is done with its split buffers
  // accumulator layout: lane holds column lane % 32, rows 8 (i / 4) + 4 (lane / 32) + i % 4
  if (bn < 24) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      part[wave][8 * (i >> 2) + 4 * bh + (i & 3)][bn] = acc[0][i] + acc[1][i];
  }
  __syncthreads();
  const int m = threadIdx.x;
  if (m < kMTok && t0 + m < T) {
    float l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) v += (part[q][m][e] + part[q][m][8 + e]) + part[q][m][16 + e];
      l[e] = v;
    }
    select_topk<8>(l, E, k, t0 + m, idx, w, logits);
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
  if (act == ACT_BF16 && E <= 8 && H % kMChunk == 0 && T >= kMfmaRouterMinTokens) {
    const dim3 grid((unsigned)((T + kMTok - 1) / kMTok));
    hipLaunchKernelGGL((router_mfma_kernel<kRouterDepth, kRouterWaves>), grid,
                       dim3(kRouterWaves * 64), 0, s,
                       static_cast<const uint16_t*>(x), wr, T, H, E, k, idx, w, logits);
    return hipGetLastError();
  }
  if (E <= 8) return launch_ec<8>(x, act, wr, T, H, E, k, idx, w, logits, s);
  return launch_ec<16>(x, act, wr, T, H, E, k, idx, w, logits, s);
}

}  // namespace moe
