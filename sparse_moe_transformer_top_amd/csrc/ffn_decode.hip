// Expert FFN for few rows per expert (decode): weight streaming.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section
// "Expert implementation: SwiGLU at scale" (w_down(silu(w_gate x) * w_up x),
// gate and up fused over the shared input) and section "Tradeoffs" (small
// expert batches leave the matrix units idle: with a handful of tokens per
// expert the layer's cost is reading the experts' weights once).
//
// With at most 16 rows per expert every weight element is used by <= 16 rows,
// so these kernels are bound by HBM: the goal is to stream each touched
// expert's weights exactly once at full bandwidth. A work-group owns 16 weight
// rows of one expert (the gate and up rows of the same 16 output columns for
// kernel 1; 16 down rows and one k split for kernel 2); its waves take the
// row's k steps round-robin, so at any time the waves of a work-group read
// neighbouring pieces of the same rows, and each lane keeps several 16-byte
// weight loads outstanding (InFlight). Weights are read in 128-byte double
// steps by nontemporal loads that each cover whole lines (dstep_operands);
// int8 and int4 rows that do not split into double steps fall back to
// 64-byte steps, whose two halves of a line are read by neighbouring waves.
// (Measured on MI355X at the Grok-1 shape: interleaved steps beat one
// contiguous k range per wave, and nontemporal loads of half lines lose
// about a quarter of the bandwidth.) The products run on
// v_mfma_f32_16x16x32_bf16 with the expert's rows as the 16-row A operand
// (rows past n_e are zero, or for int4 a repeat of the last row; neither is
// stored). The waves' partial sums are added in wave order through LDS.
// int8 weights are loaded 16 per lane (64 k per step) and converted exactly
// to bf16; their row scales multiply the float32 sums.
//
// The down projection is split over kDownSplit k ranges so that a work unit
// (16 rows x F/kDownSplit) is small against the whole launch and the last
// round of work-groups does not leave most of the GPU idle; the float32
// partials are summed in split order by a small reduce kernel.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kWavesGateUp = 16;
constexpr int kWavesDown = 8;
// int4 gate/up: 4 waves and two work-groups per CU (each wave takes twice
// the double steps of an 8-wave work-group, and one work-group fills its
// pipeline while the other drains it): 0.285 -> 0.271 ms at the Grok-1
// decode shape against 8 waves and one work-group per CU
#ifndef MOE_I4_GU_WAVES
#define MOE_I4_GU_WAVES 4
#endif
#ifndef MOE_I4_GU_WG_PER_CU
#define MOE_I4_GU_WG_PER_CU 2
#endif
// HIP reads the second __launch_bounds__ argument as a minimum number of
// waves per SIMD (amdgpu_waves_per_eu), not of work-groups per CU: W-wave
// work-groups, G per CU, are G * W / 4 waves on each of the CU's 4 SIMDs
// (two 4-wave work-groups: 2 per SIMD, a budget of 256 VGPRs per wave)
constexpr int kI4GuWavesPerSimd = MOE_I4_GU_WG_PER_CU * MOE_I4_GU_WAVES / 4;
static_assert(MOE_I4_GU_WG_PER_CU * MOE_I4_GU_WAVES % 4 == 0 && kI4GuWavesPerSimd >= 1,
              "int4 gate/up work-groups per CU must fill the 4 SIMDs evenly");
#ifndef MOE_I4_DN_WAVES
#define MOE_I4_DN_WAVES 8
#endif
// waves per work-group, by weight type
template <int WT> struct GateUpWaves { static constexpr int N = kWavesGateUp; };
template <> struct GateUpWaves<WT_I4> { static constexpr int N = MOE_I4_GU_WAVES; };
template <int WT> struct DownWaves { static constexpr int N = kWavesDown; };
template <> struct DownWaves<WT_I4> { static constexpr int N = MOE_I4_DN_WAVES; };
// int4 down: 4 k splits, so that a split's double steps (8 per wave at the
// Grok-1 shape) repay staging its group scales in LDS (stage_scales_i4);
// with 8 splits the staging was slower than reading the scales per step
#ifndef MOE_I4_DOWN_SPLIT
#define MOE_I4_DOWN_SPLIT 4
#endif
constexpr int kDownSplit = 8;
template <int WT> struct DownSplit { static constexpr int N = kDownSplit; };
template <> struct DownSplit<WT_I4> { static constexpr int N = MOE_I4_DOWN_SPLIT; };
// the workspace (decode_ws_bytes) holds kDownSplit float32 partials per row
static_assert(DownSplit<WT_BF16>::N <= kDownSplit && DownSplit<WT_I8>::N <= kDownSplit &&
                  DownSplit<WT_I4>::N <= kDownSplit,
              "a k split count above the workspace's kDownSplit partials");
// k steps each lane keeps in flight, by weight type and number of weight
// rows per lane (2: gate/up, 1: down). Measured at the Grok-1 decode shape:
// the bf16 down projection streams about 9% faster with 8 steps than with 4;
// the gate/up kernel gains nothing from 6, spills registers at 8, and is
// slower with its gate and up rows split over separate waves.
template <int WT, int NB> struct InFlight { static constexpr int N = 4; };
template <> struct InFlight<WT_BF16, 1> { static constexpr int N = 8; };
// int4 needs 64 bytes of activations per 16 bytes of weights per lane
#ifndef MOE_I4_GU_INF
#define MOE_I4_GU_INF 1
#endif
#ifndef MOE_I4_DN_INF
#define MOE_I4_DN_INF 2
#endif
template <> struct InFlight<WT_I4, 2> { static constexpr int N = MOE_I4_GU_INF; };
template <> struct InFlight<WT_I4, 1> { static constexpr int N = MOE_I4_DN_INF; };

MOE_DEV u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// A step is 64 bytes of each weight row: 32 k (bf16), 64 k (int8) or 128 k
// (int4, exactly one scale group); each lane group (lane / 16) reads 16 bytes.
template <int WT>
struct Step {
  static constexpr int K = WT == WT_I4 ? 128 : WT == WT_I8 ? 64 : 32;
  static constexpr int ESZ = WT == WT_I8 ? 1 : 2;  // weight element bytes (bf16, int8)
};

template <int WT, int NB>
MOE_DEV void mfma_step(const u32x4 (&av)[2], const u32x4 (&bv)[NB], f32x4 (&acc)[NB]) {
  if (WT == WT_I8) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const u32x4 lo = i8x8_to_bf16x8(bv[b].x, bv[b].y);
      const u32x4 hi = i8x8_to_bf16x8(bv[b].z, bv[b].w);
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

// bf16 or int8 weights: accumulate this wave's double steps of
// [d_begin, d_end) (128 bytes of each weight row: 64 k bf16, 128 k int8; the
// wave takes d_begin + wave, + W, ...) of NB 16-row weight tiles against the
// activation row arow (nullptr: zero row). wl[b][h] is this lane's load h of
// tile b at double step 0 (dstep_chunk); g = lane / 16, i = lane % 16. Each
// half of a double step is one Step<WT> (mfma_step).
template <int WT, int NB, int W, int kInFlight>
MOE_DEV void stream_dsteps(const uint16_t* arow, const char* const (&wl)[NB][2], int d_begin,
                           int d_end, int wave, int i, int g, f32x4 (&acc)[NB]) {
  constexpr int KS = Step<WT>::K;
  const int kl = WT == WT_I8 ? 16 * g : 8 * g;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int d0 = d_begin + wave; d0 < d_end; d0 += W * kInFlight) {
    u32x4 bv[kInFlight][NB][2];
    u32x4 av[kInFlight][2][2];   // [double step][half][A operand(s) of the half]
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int d = d0 + W * u;
      if (d < d_end) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int h = 0; h < 2; ++h) bv[u][b][h] = ld16_nt(wl[b][h] + (int64_t)d * 128);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = (2 * d + h) * KS + kl;
          av[u][h][0] = arow ? ldg16(arow + k) : z;
          av[u][h][1] = (WT == WT_I8 && arow) ? ldg16(arow + k + 8) : z;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      if (d0 + W * u < d_end) {
        u32x4 op[2][NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) dstep_operands(bv[u][b][0], bv[u][b][1], i, op[0][b], op[1][b]);
#pragma unroll
        for (int h = 0; h < 2; ++h) mfma_step<WT, NB>(av[u][h], op[h], acc);
      }
    }
  }
}

// This lane's two loads (dstep_chunk) of the 16-row weight tile starting at
// row n0 of a [rows][row_bytes] matrix at w (rows past the end clamped).
MOE_DEV void dstep_addrs(const void* w, int64_t n0, int64_t rows, int64_t row_bytes, int i, int g,
                         const char* (&wl)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t n = min(n0 + 8 * h + (i & 7), rows - 1);
    wl[h] = static_cast<const char*>(w) + n * row_bytes + 16 * dstep_chunk(h, i, g);
  }
}

// Accumulate this wave's steps of [s_begin, s_end) (in units of Step<WT>::K;
// the wave takes steps s_begin + wave, + W, + 2W, ...) of NB weight rows
// against the activation row arow (nullptr: zero row). Lane group g
// (lane / 16) covers 8 (bf16) or 16 (int8) consecutive k of each step.
template <int WT, int NB, int W>
MOE_DEV void stream_steps(const uint16_t* arow, const char* const (&wrow)[NB], int s_begin,
                          int s_end, int wave, int g, f32x4 (&acc)[NB]) {
  constexpr int KS = Step<WT>::K;
  constexpr int ESZ = Step<WT>::ESZ;
  constexpr int kInFlight = InFlight<WT, NB>::N;
  const int kl = WT == WT_I8 ? 16 * g : 8 * g;
  for (int s0 = s_begin + wave; s0 < s_end; s0 += W * kInFlight) {
    u32x4 bv[kInFlight][NB];
    u32x4 av[kInFlight][2];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      if (s0 + W * u < s_end) {
        const int k = (s0 + W * u) * KS + kl;
#pragma unroll
        for (int b = 0; b < NB; ++b) bv[u][b] = ldg16(wrow[b] + (int64_t)k * ESZ);
        const u32x4 z = {0u, 0u, 0u, 0u};
        av[u][0] = arow ? ldg16(arow + k) : z;
        av[u][1] = (WT == WT_I8 && arow) ? ldg16(arow + k + 8) : z;
      }
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      if (s0 + W * u < s_end) mfma_step<WT, NB>(av[u], bv[u], acc);
  }
}

// int4 weights: the same round-robin steps (one scale group each). A step's
// four MFMAs take the codes as bf16 128 + u, starting from -136 times the
// step's activations (four MFMAs against a constant operand, shared by all
// weight rows), which removes the bias (u - 8 is the value); the step's sum
// is scaled by the row's group scale into the running sums.
template <int NB, int W, int kInFlight>
MOE_DEV void stream_steps_i4(const uint16_t* arow, const char* const (&wrow)[NB],
                             const float* const (&srow)[NB], int s_begin, int s_end, int wave,
                             int g, f32x4 (&acc)[NB]) {
  constexpr uint32_t kNeg136 = 0xC308C308u;   // two bf16 -136.0
  const u32x4 cneg = {kNeg136, kNeg136, kNeg136, kNeg136};
  for (int s0 = s_begin + wave; s0 < s_end; s0 += W * kInFlight) {
    u32x4 bv[kInFlight][NB];
    u32x4 av[kInFlight][4];
    float sc[kInFlight][NB];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int s = s0 + W * u;
      if (s < s_end) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          bv[u][b] = ldg16(wrow[b] + (int64_t)s * 64 + 16 * g);
          sc[u][b] = srow[b][s];
        }
        const int k = s * 128 + 32 * g;
#pragma unroll
        for (int m = 0; m < 4; ++m) av[u][m] = ldg16(arow + k + 8 * m);
      }
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      if (s0 + W * u < s_end) {
#pragma unroll
        for (int m = 0; m < 4; ++m) av[u][m] = bf16x8_even_odd(av[u][m]);
        // -136 times the step's activations, once for all NB weight rows
        f32x4 bias = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m)
          bias = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u][m]), as_bf16x8(cneg),
                                                         bias, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const uint32_t wd[4] = {bv[u][b].x, bv[u][b].y, bv[u][b].z, bv[u][b].w};
          f32x4 t = bias;
#pragma unroll
          for (int m = 0; m < 4; ++m)
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(av[u][m]), as_bf16x8(u4x8_to_bf16x8_biased(wd[m])), t, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[b][v] = fmaf(sc[u][b], t[v], acc[b][v]);
        }
      }
    }
  }
}

// This lane's two loads (dstep_chunk) of the 16-row int4 tile starting at
// row n0 of an expert's [rows][row_bytes] matrix, as byte offsets from the
// matrix start (rows past the end clamped; the matrix is under 2 GiB).
MOE_DEV void dstep_offsets(int n0, int rows, int row_bytes, int i, int g, uint32_t (&wo)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = min(n0 + 8 * h + (i & 7), rows - 1);
    wo[h] = (uint32_t)n * (uint32_t)row_bytes + 16u * (uint32_t)dstep_chunk(h, i, g);
  }
}

// int4 weights in double steps (two scale groups, 128 bytes of each row)
// read by nontemporal full-line loads (dstep_operands): the operand of the
// first group is the lane's own load, that of the second the rotated one;
// each group as in stream_steps_i4. NM matrices (gate and up, or down) share
// the tiles' row offsets: matrix m of the expert starts at wb[m] (codes) and
// sb[m] (group scales); wo[t][h] is this lane's load h of tile t at double
// step 0 (dstep_offsets), so[t] the index of the first group scale of the
// lane's weight row in tile t (row 16 t + i). Accumulator t NM + m holds
// tile t of matrix m. The bases are uniform over the work-group, so each
// load is a scalar base plus a 32-bit lane offset. With LS the group scales
// come from the work-group's LDS table (stage_scales_i4: tile b's row r,
// group 2 d + h at scl[b ts + r ng + 2 (d - d_first) + h]); prep() runs once
// the first loads are issued (every wave calls it, also one without a double
// step).
template <int NT, int NM, int W, int kInFlight, bool LS, typename Prep>
MOE_DEV void stream_dsteps_i4(const uint16_t* arow, const char* const (&wb)[NM],
                              const uint32_t (&wo)[NT][2], const float* const (&sb)[NM],
                              const uint32_t (&so)[NT], const float* scl, int ts, int ng,
                              int d_first, int d_begin, int d_end, int wave, int i, int g,
                              f32x4 (&acc)[NT * NM], Prep prep) {
  constexpr int NB = NT * NM;
  constexpr uint32_t kNeg136 = 0xC308C308u;   // two bf16 -136.0
  const u32x4 cneg = {kNeg136, kNeg136, kNeg136, kNeg136};
  bool prepped = false;
  for (int d0 = d_begin + wave; d0 < d_end; d0 += W * kInFlight) {
    u32x4 bv[kInFlight][NB][2];
    u32x4 av[kInFlight][2][4];
    float sc[kInFlight][NB][2];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int d = d0 + W * u;
      if (d < d_end) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int m = 0; m < NM; ++m) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              bv[u][t * NM + m][h] = ld16_nt(wb[m] + (wo[t][h] + (uint32_t)d * 128u));
              if constexpr (!LS)
                sc[u][t * NM + m][h] = sb[m][so[t] + 2u * (uint32_t)d + (uint32_t)h];
            }
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = (2 * d + h) * 128 + 32 * g;
#pragma unroll
          for (int m = 0; m < 4; ++m) av[u][h][m] = ldg16(arow + k + 8 * m);
        }
      }
    }
    if (!prepped) {
      prep();
      prepped = true;
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      if (d0 + W * u < d_end) {
        if constexpr (LS) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              sc[u][b][h] = scl[b * ts + i * ng + 2 * (d0 + W * u - d_first) + h];
        }
        u32x4 op[NB][2];
#pragma unroll
        for (int b = 0; b < NB; ++b) dstep_operands(bv[u][b][0], bv[u][b][1], i, op[b][0], op[b][1]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int m = 0; m < 4; ++m) av[u][h][m] = bf16x8_even_odd(av[u][h][m]);
          f32x4 bias = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m)
            bias = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u][h][m]),
                                                           as_bf16x8(cneg), bias, 0, 0, 0);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const uint32_t wd[4] = {op[b][h].x, op[b][h].y, op[b][h].z, op[b][h].w};
            f32x4 t = bias;
#pragma unroll
            for (int m = 0; m < 4; ++m)
              t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  as_bf16x8(av[u][h][m]), as_bf16x8(u4x8_to_bf16x8_biased(wd[m])), t, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[b][v] = fmaf(sc[u][b][h], t[v], acc[b][v]);
          }
        }
      }
    }
  }  if (!prepped) prep();
}

// The same double steps as stream_dsteps_i4, software-pipelined without a
// second set of registers: right after tile b's codes of step d have been
// rearranged into MFMA operands (dstep_operands), the loads of tile b for
// the wave's next step go into the same registers, so the wave's next step
// streams in while it converts and multiplies the rest of step d (the
// conversion's VALU work is about half the time the loads take). The last
// step is peeled, so every load in the loop is unconditional.
// Group scales: with LS from the work-group's LDS table (stage_scales_i4:
// tile b's row r, group c at scl[b ts + r G + c]), all of a step's read at
// its start; otherwise from global memory, each loaded one step ahead.
// prep() runs once the first step's loads are issued (every wave calls it,
// also one without a double step).
template <int NT, int NM, int W, bool LS, typename Prep>
MOE_DEV void stream_dsteps_i4_roll(const uint16_t* arow, const char* const (&wb)[NM],
                                   const uint32_t (&wo)[NT][2], const float* const (&sb)[NM],
                                   const uint32_t (&so)[NT], const float* scl, int ts, int G,
                                   int d_begin, int d_end, int wave, int i, int g,
                                   f32x4 (&acc)[NT * NM], Prep prep) {
  constexpr int NB = NT * NM;
  constexpr uint32_t kNeg136 = 0xC308C308u;   // two bf16 -136.0
  const u32x4 cneg = {kNeg136, kNeg136, kNeg136, kNeg136};
  int d = d_begin + wave;
  if (d >= d_end) {
    prep();
    return;
  }
  u32x4 bv[NB][2];
  float2 sc[NB];   // the two group scales of a double step
  u32x4 av[2][4];
  auto load_w = [&](int t, int m, int dd) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      bv[t * NM + m][h] = ld16_nt(wb[m] + (wo[t][h] + (uint32_t)dd * 128u));
  };
  auto load_s = [&](int t, int m, int dd) {
    if constexpr (!LS) {
      const float* p = sb[m] + so[t] + 2u * (uint32_t)dd;   // scale arrays are only 4-byte aligned
      sc[t * NM + m] = make_float2(p[0], p[1]);
    }
  };
  auto load_a = [&](int dd) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < 4; ++m) av[h][m] = ldg16(arow + (2 * dd + h) * 128 + 32 * g + 8 * m);
  };
  load_a(d);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      load_w(t, m, d);
      load_s(t, m, d);
    }
  prep();
  // one double step from the registers; with more, the loads of step dn
  // replace each operand as soon as it has been consumed
  auto step = [&](auto more, int dc, int dn) {
    if constexpr (LS) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        sc[b] = *reinterpret_cast<const float2*>(scl + b * ts + i * G + 2 * dc);
    }
    u32x4 a[2][4];
    f32x4 bias[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bias[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        a[h][m] = bf16x8_even_odd(av[h][m]);
        bias[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[h][m]), as_bf16x8(cneg),
                                                          bias[h], 0, 0, 0);
      }
    }
    if constexpr (decltype(more)::value) load_a(dn);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int b = t * NM + m;
        u32x4 op[2];
        dstep_operands(bv[b][0], bv[b][1], i, op[0], op[1]);
        if constexpr (decltype(more)::value) load_w(t, m, dn);
        const float s[2] = {sc[b].x, sc[b].y};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t wd[4] = {op[h].x, op[h].y, op[h].z, op[h].w};
          f32x4 r = bias[h];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(a[h][q]), as_bf16x8(u4x8_to_bf16x8_biased(wd[q])), r, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[b][v] = fmaf(s[h], r[v], acc[b][v]);
        }
        // the scales are loaded once used, so no copy of them is kept
        if constexpr (decltype(more)::value) load_s(t, m, dn);
        // keep the tiles in order: hoisting a later tile's operand
        // rearrangement would wait for all of the step's loads
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (; d + W < d_end; d += W) step(std::true_type{}, d, d + W);
  step(std::false_type{}, d, 0);
}

// 64 lanes x 4 bytes from global memory (per-lane address) into LDS at byte
// address lds + 4 lane (lds wave-uniform); writes no VGPR. The caller waits
// for it with s_waitcnt vmcnt before the LDS is read.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
MOE_DEV void lds_dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
typedef __attribute__((address_space(3))) void lds_void_t;
MOE_DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void_t*)p; }

// The int4 group scales a work-group's NB 16-row tiles need, staged in LDS
// by direct-to-LDS loads at the start of the kernel. Read from global memory
// at each double step, a tile's 2 scales of 16 rows touch 16 cache lines for
// 128 useful bytes, about as many L2 requests as the weight stream itself;
// staged once, the gate/up stream takes ~10% less time and the down
// projection ~7% at the Grok-1 shape. Tile b's row r holds ng groups (the
// work-group's range: all G of a gate/up row, a k split's of a down row;
// tile0[b] points at row 0's first group of the range, rows G apart) at
// scl[b ts + r ng + c], ts = 16 ng rounded up to 64 floats. The table is
// copied in 256-byte pieces (64 lanes x 4 bytes, each lane its own source
// address; for a whole row, 16 consecutive rows are contiguous), round-robin
// over the waves; lanes past a tile's last scale read that scale again (in
// bounds) into the stride's padding. No wait here: the stream's prep waits
// for the loads and synchronises the block.
constexpr int kI4ScaleTable = 1024;   // floats per tile in the table: 16 rows of <= 64 groups
__host__ __device__ inline int scale_tile_stride(int ng) { return (16 * ng + 63) / 64 * 64; }
// s_waitcnt vmcnt(0), leaving the other counters untouched
MOE_DEV void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00); }
template <int NB, int W>
MOE_DEV void stage_scales_i4(float* scl, int ts, int ng, int G, const float* const (&tile0)[NB],
                             int wave, int lane) {
  const int pieces = ts / 64, n = 16 * ng;
  for (int q = wave; q < NB * pieces; q += W) {
    const int b = q / pieces, f = (q - b * pieces) * 64 + lane, fc = min(f, n - 1);
    lds_dma4(tile0[b] + (ng == G ? fc : (fc / ng) * G + fc % ng),
             __builtin_amdgcn_readfirstlane(lds_addr(scl) + (uint32_t)(b * ts + f - lane) * 4u));
  }
}

// contiguous share [b, e) of n steps for part p of parts
MOE_DEV void split_range(int n, int parts, int p, int& b, int& e) {
  const int q = (n + parts - 1) / parts;
  b = min(n, p * q);
  e = min(n, b + q);
}

// Kernel 1: h = silu(x W_gate^T) * (x W_up^T) for <= 16 rows per expert.
template <int WT>
__global__ __launch_bounds__(GateUpWaves<WT>::N * 64) void gateup_decode_kernel(FfnArgs a) {
  constexpr int kWaves = GateUpWaves<WT>::N;
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
  f32x4 acc[2];
  acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc[1] = acc[0];
  if (WT == WT_BF16 || (WT == WT_I8 && a.H % 128 == 0)) {
    // full-line double steps of 128 bytes per row
    const char* wl[2][2];
    const int64_t r0w = (int64_t)e * a.F;   // the expert's first weight row
    const int64_t rb = (int64_t)a.H * Step<WT>::ESZ;
    dstep_addrs(a.wg, r0w + n0, r0w + a.F, rb, i, g, wl[0]);
    dstep_addrs(a.wu, r0w + n0, r0w + a.F, rb, i, g, wl[1]);
    stream_dsteps<WT, 2, kWaves, InFlight<WT, 2>::N / 2>(arow, wl, 0, (int)(rb / 128), wave, i, g,
                                                         acc);
  } else {
    const int64_t roff = ((int64_t)e * a.F + n) * a.H * Step<WT>::ESZ;
    const char* const wrow[2] = {static_cast<const char*>(a.wg) + roff,
                                 static_cast<const char*>(a.wu) + roff};
    stream_steps<WT, 2, kWaves>(arow, wrow, 0, a.H / Step<WT>::K, wave, g, acc);
  }

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

// Kernel 2: float32 partial sums of y = h W_down^T over one k split, for
// <= 16 rows per expert: part[split][row][H].
template <int WT>
__global__ __launch_bounds__(DownWaves<WT>::N * 64) void down_decode_kernel(FfnArgs a) {
  constexpr int kWaves = DownWaves<WT>::N;
  __shared__ float red[kWaves][4][64];
  const int nt_per_e = (a.H + 15) / 16;
  constexpr int kSplit = DownSplit<WT>::N;
  const int split = blockIdx.x % kSplit;
  const int tile = blockIdx.x / kSplit;
  const int e = tile / nt_per_e;
  const int n0 = (tile % nt_per_e) * 16;
  const int r0 = a.offsets[e];
  const int ne = a.offsets[e + 1] - r0;
  if (ne <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const uint16_t* arow = i < ne ? static_cast<const uint16_t*>(a.h) + (int64_t)(r0 + i) * a.F
                                : nullptr;
  const int n = min(n0 + i, a.H - 1);
  f32x4 acc[1];
  acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  int kb, ke;
  if (WT == WT_BF16 || (WT == WT_I8 && a.F % 128 == 0)) {
    const int64_t rb = (int64_t)a.F * Step<WT>::ESZ;
    split_range((int)(rb / 128), kSplit, split, kb, ke);
    const char* wl[1][2];
    const int64_t r0w = (int64_t)e * a.H;
    dstep_addrs(a.wd, r0w + n0, r0w + a.H, rb, i, g, wl[0]);
    stream_dsteps<WT, 1, kWaves, InFlight<WT, 1>::N / 2>(arow, wl, kb, ke, wave, i, g, acc);
  } else {
    split_range(a.F / Step<WT>::K, kSplit, split, kb, ke);
    const char* const wrow[1] = {static_cast<const char*>(a.wd) +
                                 ((int64_t)e * a.H + n) * a.F * Step<WT>::ESZ};
    stream_steps<WT, 1, kWaves>(arow, wrow, kb, ke, wave, g, acc);
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][v][lane] = acc[0][v];
  __syncthreads();
  if (wave != 0) return;
  const int col = n0 + i;
  if (col >= a.H) return;
  float* part = static_cast<float*>(a.ws) + (int64_t)split * a.T * a.k * a.H;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * g + v;
    if (row >= ne) continue;
    float ys = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ys += red[w][v][lane];
    if (WT == WT_I8) ys *= a.sd[(int64_t)e * a.H + col];
    part[(int64_t)(r0 + row) * a.H + col] = ys;
  }
}

// int4 weights: a work-group covers NT tiles of 16 output columns. A lane's
// activation chunks (64 bytes for the 32 codes of each 16-byte weight load)
// then serve the weight rows of all NT tiles, which cuts the activation
// requests per weight byte by NT (with int4 codes the activations, 2 bytes
// per code against half a byte of weight, were two thirds of the bytes a
// work-group requested). Measured at the Grok-1 decode shape (T = 8) with
// 64-byte steps: two tiles with one step in flight per lane for gate/up
// (0.427 ms against 0.441 for one tile with two steps; four tiles, or two
// with two steps, cost occupancy and were slower), two tiles with two steps
// for down (0.224 ms against 0.266 for one tile with four). With full-line
// double steps (stream_dsteps_i4, when the scale-group count is even): one
// double step in flight, gate/up 0.354 ms and down 0.185 ms; then four
// tiles for gate/up (the kernel then ran one 8-wave work-group per CU, so
// the extra registers cost no occupancy) 0.326 ms; one tile was within
// noise, two double steps in flight, or four tiles for down, were slower.
// With the pipelined stream and 4-wave work-groups, three tiles equal four.
#ifndef MOE_I4_GU_NT
#define MOE_I4_GU_NT 2
#endif
#ifndef MOE_I4_GU_NT_FULL
#define MOE_I4_GU_NT_FULL 4
#endif
#ifndef MOE_I4_DN_NT
#define MOE_I4_DN_NT 2
#endif
constexpr int kI4GateUpTiles = MOE_I4_GU_NT;            // 64-byte steps
constexpr int kI4GateUpTilesFull = MOE_I4_GU_NT_FULL;   // full-line double steps
constexpr int kI4DownTiles = MOE_I4_DN_NT;

template <int NT, bool LS>
__global__ __launch_bounds__(GateUpWaves<WT_I4>::N * 64, kI4GuWavesPerSimd) void gateup_decode_i4_kernel(FfnArgs a) {
  constexpr int kWaves = GateUpWaves<WT_I4>::N;
  static_assert(NT <= kWaves, "one wave per tile in the epilogue");
  __shared__ float red[kWaves][2 * NT][4][64];
  __shared__ __align__(16) float scl[LS ? 2 * NT * kI4ScaleTable : 1];
  const int groups = (a.F + 16 * NT - 1) / (16 * NT);
  const int e = blockIdx.x / groups;
  const int n0 = (blockIdx.x % groups) * 16 * NT;
  const int r0 = a.offsets[e];
  const int ne = a.offsets[e + 1] - r0;
  if (ne <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  // lanes past the expert's rows repeat its last row: their output rows
  // are never stored, and every lane's loads stay unconditional
  const uint16_t* arow =
      static_cast<const uint16_t*>(a.x) + (int64_t)(a.perm[r0 + min(i, ne - 1)] / a.k) * a.H;
  const char* wrow[2 * NT];
  const float* srow[2 * NT];
  f32x4 acc[2 * NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t row = (int64_t)e * a.F + min(n0 + 16 * t + i, a.F - 1);
    wrow[2 * t] = static_cast<const char*>(a.wg) + row * (a.H / 2);
    wrow[2 * t + 1] = static_cast<const char*>(a.wu) + row * (a.H / 2);
    srow[2 * t] = a.sg + row * (a.H / 128);
    srow[2 * t + 1] = a.su + row * (a.H / 128);
    acc[2 * t] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[2 * t + 1] = acc[2 * t];
  }
  if ((a.H / 128) % 2 == 0) {
    // full-line double steps (two scale groups)
    const int64_t eb = (int64_t)e * a.F * (a.H / 2), es = (int64_t)e * a.F * (a.H / 128);
    const char* wb[2] = {static_cast<const char*>(a.wg) + eb, static_cast<const char*>(a.wu) + eb};
    const float* sb[2] = {a.sg + es, a.su + es};
    uint32_t wo[NT][2], so[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      dstep_offsets(n0 + 16 * t, a.F, a.H / 2, i, g, wo[t]);
      so[t] = (uint32_t)min(n0 + 16 * t + i, a.F - 1) * (uint32_t)(a.H / 128);
    }
    const int G = a.H / 128, ts = scale_tile_stride(G);
    if constexpr (LS) {   // G <= 64 (checked at launch)
      const float* tile0[2 * NT];
#pragma unroll
      for (int b = 0; b < 2 * NT; ++b) tile0[b] = sb[b % 2] + (int64_t)(n0 + 16 * (b / 2)) * G;
      stage_scales_i4<2 * NT, kWaves>(scl, ts, G, G, tile0, wave, lane);
    }
    auto prep = [&]() {
      if constexpr (LS) {   // the staged scales (and the first step's loads) landed
        wait_vmcnt0();
        __syncthreads();
      }
    };
    stream_dsteps_i4_roll<NT, 2, kWaves, LS>(arow, wb, wo, sb, so, scl, ts, G, 0, a.H / 256,
                                             wave, i, g, acc, prep);
  } else {
    stream_steps_i4<2 * NT, kWaves, InFlight<WT_I4, 2>::N>(arow, wrow, srow, 0, a.H / 128, wave,
                                                           g, acc);
  }
#pragma unroll
  for (int b = 0; b < 2 * NT; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][b][v][lane] = acc[b][v];
  __syncthreads();
  // wave t writes tile t (t < NT), summing the waves' partials in wave order
  if (wave >= NT) return;
  const int col = n0 + 16 * wave + i;
  if (col >= a.F) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * g + v;
    if (row >= ne) continue;
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      gs += red[w][2 * wave][v][lane];
      us += red[w][2 * wave + 1][v][lane];
    }
    static_cast<uint16_t*>(a.h)[(int64_t)(r0 + row) * a.F + col] = f32_to_bf16_bits(swiglu(gs, us));
  }
}

template <int NT, bool LS>
__global__ __launch_bounds__(DownWaves<WT_I4>::N * 64) void down_decode_i4_kernel(FfnArgs a) {
  constexpr int kWaves = DownWaves<WT_I4>::N;
  constexpr int kSplit = DownSplit<WT_I4>::N;
  static_assert(NT <= kWaves, "one wave per tile in the epilogue");
  __shared__ float red[kWaves][NT][4][64];
  __shared__ __align__(16) float scl[LS ? NT * kI4ScaleTable : 1];
  const int groups = (a.H + 16 * NT - 1) / (16 * NT);
  const int split = blockIdx.x % kSplit;
  const int tile = blockIdx.x / kSplit;
  const int e = tile / groups;
  const int n0 = (tile % groups) * 16 * NT;
  const int r0 = a.offsets[e];
  const int ne = a.offsets[e + 1] - r0;
  if (ne <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  // lanes past the expert's rows repeat its last row (never stored)
  const uint16_t* arow = static_cast<const uint16_t*>(a.h) + (int64_t)(r0 + min(i, ne - 1)) * a.F;
  const char* wrow[NT];
  const float* srow[NT];
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t row = (int64_t)e * a.H + min(n0 + 16 * t + i, a.H - 1);
    wrow[t] = static_cast<const char*>(a.wd) + row * (a.F / 2);
    srow[t] = a.sd + row * (a.F / 128);
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int kb, ke;
  if ((a.F / 128) % 2 == 0) {
    split_range(a.F / 256, kSplit, split, kb, ke);
    const char* wb[1] = {static_cast<const char*>(a.wd) + (int64_t)e * a.H * (a.F / 2)};
    const float* sb[1] = {a.sd + (int64_t)e * a.H * (a.F / 128)};
    uint32_t wo[NT][2], so[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      dstep_offsets(n0 + 16 * t, a.H, a.F / 2, i, g, wo[t]);
      so[t] = (uint32_t)min(n0 + 16 * t + i, a.H - 1) * (uint32_t)(a.F / 128);
    }
    // the split's groups [2 kb, 2 ke) of the tiles' rows (at most 64: checked at launch)
    const int G = a.F / 128, ng = 2 * (ke - kb), ts = scale_tile_stride(ng);
    if constexpr (LS) {
      if (ng > 0) {
        const float* tile0[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) tile0[t] = sb[0] + (int64_t)(n0 + 16 * t) * G + 2 * kb;
        stage_scales_i4<NT, kWaves>(scl, ts, ng, G, tile0, wave, lane);
      }
    }
    auto prep = [&]() {
      if constexpr (LS) {   // the staged scales (and the first step's loads) landed
        wait_vmcnt0();
        __syncthreads();
      }
    };
    // (the pipelined stream, stream_dsteps_i4_roll, needs 163 VGPRs here
    // against 121, which halves the work-groups per CU: measured slower)
    stream_dsteps_i4<NT, 1, kWaves, (InFlight<WT_I4, 1>::N + 1) / 2, LS>(
        arow, wb, wo, sb, so, scl, ts, ng, kb, kb, ke, wave, i, g, acc, prep);
  } else {
    split_range(a.F / 128, kSplit, split, kb, ke);
    stream_steps_i4<NT, kWaves, InFlight<WT_I4, 1>::N>(arow, wrow, srow, kb, ke, wave, g, acc);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][t][v][lane] = acc[t][v];
  __syncthreads();
  if (wave >= NT) return;
  const int col = n0 + 16 * wave + i;
  if (col >= a.H) return;
  float* part = static_cast<float*>(a.ws) + (int64_t)split * a.T * a.k * a.H;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * g + v;
    if (row >= ne) continue;
    float ys = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ys += red[w][wave][v][lane];
    part[(int64_t)(r0 + row) * a.H + col] = ys;
  }
}

// y[r, :] = bf16(sum over splits of part[split][r][:]) for r < offsets[E].
__global__ __launch_bounds__(256) void down_reduce_kernel(FfnArgs a, int nsplit) {
  const int chunks = a.H / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gid / chunks;
  if (r >= a.offsets[a.E]) return;
  const int c = (int)(gid - r * chunks) * 4;
  const float* part = static_cast<const float*>(a.ws);
  const int64_t stride = a.T * a.k * a.H;
  float4 s = *reinterpret_cast<const float4*>(part + r * a.H + c);
#pragma unroll
  for (int p = 1; p < nsplit; ++p) {
    const float4 v = *reinterpret_cast<const float4*>(part + p * stride + r * a.H + c);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  uint2 o;
  o.x = pack_bf16x2(s.x, s.y);
  o.y = pack_bf16x2(s.z, s.w);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + r * a.H + c) = o;
}

}  // namespace

size_t decode_ws_bytes(int64_t T, int H, int k) {
  return (size_t)kDownSplit * T * k * H * sizeof(float);
}

hipError_t launch_gateup_decode(const FfnArgs& a, Wt wt, hipStream_t s) {
  // up to 8 tokens with bf16 weights: the LDS-staged kernel (ffn_decode_lds.hip)
  const hipError_t e = launch_gateup_decode_lds(a, wt, s);
  if (e != hipErrorNotSupported) return e;
  const dim3 grid((unsigned)(a.E * ((a.F + 15) / 16)));
  if (wt == WT_I8)
    hipLaunchKernelGGL(gateup_decode_kernel<WT_I8>, grid, dim3(GateUpWaves<WT_I8>::N * 64), 0, s,
                       a);
  else if (wt == WT_I4 && (a.H / 128) % 2 == 0) {   // the kernel takes double steps
    const dim3 g4((unsigned)(a.E * ((a.F + 16 * kI4GateUpTilesFull - 1) /
                                    (16 * kI4GateUpTilesFull))));
    if (scale_tile_stride(a.H / 128) <= kI4ScaleTable)   // the LDS scale table holds them
      hipLaunchKernelGGL((gateup_decode_i4_kernel<kI4GateUpTilesFull, true>), g4,
                         dim3(GateUpWaves<WT_I4>::N * 64), 0, s, a);
    else
      hipLaunchKernelGGL((gateup_decode_i4_kernel<kI4GateUpTilesFull, false>), g4,
                         dim3(GateUpWaves<WT_I4>::N * 64), 0, s, a);
  } else if (wt == WT_I4)
    hipLaunchKernelGGL((gateup_decode_i4_kernel<kI4GateUpTiles, false>),
                       dim3((unsigned)(a.E * ((a.F + 16 * kI4GateUpTiles - 1) /
                                              (16 * kI4GateUpTiles)))),
                       dim3(GateUpWaves<WT_I4>::N * 64), 0, s, a);
  else
    hipLaunchKernelGGL(gateup_decode_kernel<WT_BF16>, grid, dim3(GateUpWaves<WT_BF16>::N * 64), 0,
                       s, a);
  return hipGetLastError();
}

hipError_t launch_down_decode(const FfnArgs& a, Wt wt, hipStream_t s) {
  const auto grid = [&](int nsplit) {
    return dim3((unsigned)(a.E * ((a.H + 15) / 16) * nsplit));
  };
  int nsplit = kDownSplit;
  if (wt == WT_I8) {
    hipLaunchKernelGGL(down_decode_kernel<WT_I8>, grid(DownSplit<WT_I8>::N),
                       dim3(DownWaves<WT_I8>::N * 64), 0, s, a);
    nsplit = DownSplit<WT_I8>::N;
  } else if (wt == WT_I4) {
    const unsigned groups = (unsigned)((a.H + 16 * kI4DownTiles - 1) / (16 * kI4DownTiles));
    const dim3 gd((unsigned)a.E * groups * DownSplit<WT_I4>::N);
    // a split's double steps: at most ceil(F / 256 / splits), two groups each
    const int dsteps = (a.F / 256 + DownSplit<WT_I4>::N - 1) / DownSplit<WT_I4>::N;
    if ((a.F / 128) % 2 == 0 && scale_tile_stride(2 * dsteps) <= kI4ScaleTable)
      hipLaunchKernelGGL((down_decode_i4_kernel<kI4DownTiles, true>), gd,
                         dim3(DownWaves<WT_I4>::N * 64), 0, s, a);
    else
      hipLaunchKernelGGL((down_decode_i4_kernel<kI4DownTiles, false>), gd,
                         dim3(DownWaves<WT_I4>::N * 64), 0, s, a);
    nsplit = DownSplit<WT_I4>::N;
  } else {
    hipLaunchKernelGGL(down_decode_kernel<WT_BF16>, grid(DownSplit<WT_BF16>::N),
                       dim3(DownWaves<WT_BF16>::N * 64), 0, s, a);
    nsplit = DownSplit<WT_BF16>::N;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t items = a.T * a.k * (a.H / 4);
  hipLaunchKernelGGL(down_reduce_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s,
                     a, nsplit);
  return hipGetLastError();
}

}  // namespace moe
