// Internal launcher interface between the C ABI (capi.cpp) and the kernels.
// Launchers assume their arguments were validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum Act { ACT_F32 = 0, ACT_BF16 = 1 };
enum Wt { WT_F32 = 0, WT_BF16 = 1, WT_I8 = 2, WT_I4 = 3 };

// router.hip
hipError_t launch_router_topk(const void* x, Act act, const float* wr, int64_t T, int H,
                              int E, int k, int32_t* idx, float* w, float* logits,
                              hipStream_t s);

// dispatch.hip
size_t dispatch_ws_bytes(int64_t T, int E);
hipError_t launch_dispatch(const int32_t* idx, int64_t T, int E, int k, int64_t cap,
                           int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* slot_row, uint8_t* dropped, void* ws, hipStream_t s);

// fills n int32 values with v (a kernel, so it is safe inside captured graphs)
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);

// combine.hip
hipError_t launch_combine(const void* y_perm, const int32_t* slot_row, const float* w,
                          int64_t T, int H, int k, Act act, void* out, hipStream_t s);

// ffn_*.hip: expert FFN over dispatched rows
struct FfnArgs {
  const void* x;          // [T,H] act
  const int32_t* perm;    // [T*k]
  const int32_t* offsets; // [E+1]
  int64_t T;
  int H, F, E, k;
  const void* wg;         // [E,F,H] (int4: [E,F,H/2] bytes, two codes per byte)
  const void* wu;         // [E,F,H]
  const void* wd;         // [E,H,F] (int4: [E,H,F/2])
  const float* sg;        // int8: [E,F] row scales; int4: [E,F,H/128] group scales
  const float* su;        // as sg
  const float* sd;        // int8: [E,H]; int4: [E,H,F/128]
  void* h;                // [T*k,F] act
  void* y;                // [T*k,H] act
  void* ws;               // decode: split-k partials; tiled down: tail partials
  void* g_save;           // [T*k,F] bf16 pre-activations (launch_gateup_save_tiled only)
  void* u_save;           // [T*k,F]
};

// largest T for which the decode (few rows per expert) kernels are used
constexpr int64_t kDecodeMaxT = 16;
// gate/up with the expert's token rows in LDS (ffn_decode_lds.hip, bf16
// weights): up to this many tokens, when their rows fit one work-group's LDS
constexpr int64_t kDecodeLdsMaxT = 8;
constexpr size_t kDecodeLdsMax = 160 * 1024;
size_t decode_lds_bytes(int64_t T, int H);
// hipErrorNotSupported (nothing launched) when T or the LDS need is too large
hipError_t launch_gateup_decode_lds(const FfnArgs& a, Wt wt, hipStream_t s);

size_t ffn_ws_bytes(int64_t T, int H, int F, int E, int k, Act act, Wt wt);
// scratch of a tiled down-mode launch (float32 partials of its split tail tiles)
size_t tiled_ws_bytes();
// gate/up product with the SwiGLU epilogue (writes h) and down product (writes y)
hipError_t launch_gateup_f32(const FfnArgs& a, hipStream_t s);
hipError_t launch_down_f32(const FfnArgs& a, hipStream_t s);
hipError_t launch_gateup_tiled(const FfnArgs& a, Wt wt, hipStream_t s);
hipError_t launch_down_tiled(const FfnArgs& a, Wt wt, hipStream_t s);
// bf16 gate/up that also writes g_save and u_save (training forward)
hipError_t launch_gateup_save_tiled(const FfnArgs& a, hipStream_t s);

// Weight gradients on row-major operands (ffn_tiled.hip): per expert e,
// C_e[m][n] = sum over e's dispatch rows r of a[r][m] * b[r][n]. a and b
// must stay readable for 63 rows past the last dispatch row (those rows are
// read and masked out).
struct WgradTnArgs {
  const void* a;          // [rows][lda] bf16
  int64_t lda;            // elements per row of a (>= M)
  const void* b;          // [rows][ldb] bf16
  int64_t ldb;            // elements per row of b (>= N)
  const int32_t* offsets; // [E+1] dispatch offsets
  int E, M, N, m_split;   // M, N multiples of 64
  void* out0;             // [E][m_split][N] bf16
  void* out1;             // [E][M - m_split][N] bf16 (unused when m_split == M)
  int m_fast;             // 1: tiles sharing a B block run together
};
hipError_t launch_wgrad_tn(const WgradTnArgs& w, hipStream_t s);

// Data gradients on the stored weights (ffn_tiled.hip): for every expert's
// dispatch rows r, y[r][n] = sum_k a[r][k] W_e[k][n], W_e[k] row k of b0[e]
// ([ksplit][N]) for k < ksplit, else row k - ksplit of b1[e] ([K-ksplit][N]).
struct DgradArgs {
  const void* a;          // [T*k][K] bf16
  const int32_t* offsets; // [E+1]
  int64_t T;
  int E, k;
  int N, K, ksplit;       // multiples of 64
  const void* b0;
  const void* b1;         // may be null when ksplit == K
  void* y;                // [T*k][N] bf16
  void* ws;               // tiled_ws_bytes() of scratch (split tail tiles)
};
hipError_t launch_dgrad_nn(const DgradArgs& d, hipStream_t s);
size_t decode_ws_bytes(int64_t T, int H, int k);
hipError_t launch_gateup_decode(const FfnArgs& a, Wt wt, hipStream_t s);
hipError_t launch_down_decode(const FfnArgs& a, Wt wt, hipStream_t s);

// noalloc.hip: device address of the library's fixed scratch array
// (MOE_NOALLOC_SCRATCH_BYTES) on the current device, looked up once per device
hipError_t noalloc_scratch(void** ptr);

// routing statistics (stats.hip)
hipError_t launch_routing_stats(const float* logits, const int32_t* counts, int64_t T, int E,
                                int k, float* util, float* margin, float* mass, hipStream_t s);

// backward of the layer (bwd.hip), bf16 activations and weights
int64_t router_wgrad_chunks(int64_t T);
hipError_t launch_combine_bwd(const void* dout, const void* y, const int32_t* slot_row,
                              const float* w, const int32_t* idx, int64_t T, int H, int E, int k,
                              void* dy, float* dw, float* dl, hipStream_t s);
hipError_t launch_swiglu_bwd(const void* dh, const void* g, const void* u, const int32_t* offsets,
                             int E, int64_t max_rows, int F, void* dgu, hipStream_t s);
hipError_t launch_dx_combine(const void* dxr, const int32_t* slot_row, const int32_t* idx,
                             const float* dl, const float* wr, int64_t T, int H, int E, int k,
                             void* dx, hipStream_t s);
// part: router_wgrad_chunks(T) * E * H floats
hipError_t launch_router_wgrad(const void* x, const float* dl, int64_t T, int H, int E,
                               float* part, float* dwr, hipStream_t s);

// expert-parallel layouts (ep.hip)
hipError_t launch_ep_pack(const void* x, int64_t row_bytes, const int32_t* perm,
                          const int32_t* offsets, int64_t max_rows, int E, int k, int R,
                          void* send, int32_t* send_counts, hipStream_t s);
hipError_t launch_ep_recv_layout(const int32_t* counts, int R, int El, int64_t max_rows,
                                 int32_t* offsets, int32_t* row_index, hipStream_t s);
hipError_t launch_ep_unpack(const void* y, int64_t row_bytes, const int32_t* row_index,
                            const int32_t* offsets, int El, int64_t max_rows, void* back,
                            hipStream_t s);

}  // namespace moe
