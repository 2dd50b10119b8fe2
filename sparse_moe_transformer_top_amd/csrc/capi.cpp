// C ABI of the top-2 MoE FFN layer: argument checks, workspace layout and
// kernel launches. The contract of every entry point is in include/moe.h.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kernels.h"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t act_size(moe_dtype d) { return d == MOE_F32 ? 4 : 2; }

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

moe_status check_shape(int64_t T, int32_t E, int32_t k) {
  REQUIRE(T >= 0, MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 (got %lld)", (long long)T);
  REQUIRE(E >= 1 && k >= 1 && k <= E, MOE_ERR_INVALID_ARGUMENT,
          "need 1 <= k <= E (got E=%d k=%d)", E, k);
  REQUIRE(E <= 16, MOE_ERR_UNSUPPORTED, "E=%d > 16 experts is not supported", E);
  REQUIRE(k <= 4, MOE_ERR_UNSUPPORTED, "k=%d > 4 is not supported", k);
  REQUIRE(T * (int64_t)k < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED,
          "T*k=%lld does not fit int32 row indices", (long long)(T * k));
  return ok();
}

moe_status check_dim(const char* name, int32_t v) {
  REQUIRE(v >= 1, MOE_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %d)", name, v);
  REQUIRE(v % 64 == 0, MOE_ERR_UNSUPPORTED, "%s=%d must be a multiple of 64", name, v);
  REQUIRE(v <= (1 << 20), MOE_ERR_UNSUPPORTED, "%s=%d is above the supported 1048576", name, v);
  return ok();
}

moe_status check_act(moe_dtype a) {
  REQUIRE(a == MOE_F32 || a == MOE_BF16, MOE_ERR_UNSUPPORTED,
          "activation dtype %d: only MOE_F32 and MOE_BF16 are supported", (int)a);
  return ok();
}

moe_status check_pair(moe_dtype act, moe_dtype w) {
  moe_status s = check_act(act);
  if (s) return s;
  const bool good = (act == MOE_F32 && w == MOE_F32) ||
                    (act == MOE_BF16 && (w == MOE_BF16 || w == MOE_I8 || w == MOE_I4));
  REQUIRE(good, MOE_ERR_UNSUPPORTED,
          "unsupported (activation, weight) dtypes (%d, %d): use (F32,F32), (BF16,BF16), "
          "(BF16,I8) or (BF16,I4)", (int)act, (int)w);
  return ok();
}

// int4 weights: decode kernels only (T <= kDecodeMaxT), scale groups of 128 k
moe_status check_int4(int64_t T, int32_t H, int32_t F, moe_dtype w) {
  if (w != MOE_I4) return ok();
  REQUIRE(T <= kDecodeMaxT, MOE_ERR_UNSUPPORTED,
          "MOE_I4 weights are supported for T <= %lld (decode), got T=%lld",
          (long long)kDecodeMaxT, (long long)T);
  REQUIRE(H % 128 == 0 && F % 128 == 0, MOE_ERR_UNSUPPORTED,
          "MOE_I4 weights need H and F multiples of 128 (got H=%d F=%d)", H, F);
  // the kernels address one expert's codes with 32-bit offsets
  REQUIRE((int64_t)H * F / 2 < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED,
          "MOE_I4 weights need an expert matrix under 2 GiB (H*F/2 < 2^31, got H=%d F=%d)", H,
          F);
  return ok();
}

bool has_scales(moe_dtype w) { return w == MOE_I8 || w == MOE_I4; }

int64_t capacity_of(int64_t T, int32_t k, int32_t E, float cf) {
  if (!(cf > 0.0f) || std::isinf(cf)) return -1;
  return (int64_t)std::ceil((double)cf * (double)(T * k) / (double)E);
}

struct LayerWs {
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* slot_row;
  uint8_t* dropped;
  void* dws;
  void* h;
  void* y;
  void* fws;
  size_t total;
};

LayerWs layer_ws_layout(char* base, int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                        moe_dtype act, moe_dtype wt) {
  LayerWs L{};
  const int64_t N = T * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return static_cast<void*>(p);
  };
  L.idx = static_cast<int32_t*>(take(N * 4));
  L.w = static_cast<float*>(take(N * 4));
  L.counts = static_cast<int32_t*>(take(E * 4));
  L.offsets = static_cast<int32_t*>(take((E + 1) * 4));
  L.perm = static_cast<int32_t*>(take(N * 4));
  L.slot_row = static_cast<int32_t*>(take(N * 4));
  L.dropped = static_cast<uint8_t*>(take(N));
  L.dws = take(dispatch_ws_bytes(T, E));
  L.h = take((size_t)N * F * act_size(act));
  L.y = take((size_t)N * H * act_size(act));
  L.fws = take(ffn_ws_bytes(T, H, F, E, k, act == MOE_F32 ? ACT_F32 : ACT_BF16, (Wt)wt));
  L.total = off;
  return L;
}

// The weight-gradient kernel reads up to 63 rows past an expert's last
// dispatch row (and masks them out), so the buffers it reads (h in the
// reserve; dy, [dg | du] and the gathered x in the backward scratch) keep
// kBwdSlackRows rows after row T*k.
constexpr int64_t kBwdSlackRows = 64;

// The training reserve (written by moe_layer_forward_train, read by
// moe_layer_backward); the order is part of the ABI (include/moe.h).
struct TrainReserve {
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* slot_row;
  uint8_t* dropped;
  void* dws;
  void* fws;    // tile scratch of the down projection
  void* g;
  void* u;
  void* h;
  void* y;
  size_t total;
};

// Consecutive 256-byte-aligned pieces of one buffer (sizes only when base is NULL).
struct Carver {
  char* base;
  size_t off;
  void* take(size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  }
};

TrainReserve train_reserve_layout(char* base, int64_t T, int32_t H, int32_t F, int32_t E,
                                  int32_t k) {
  TrainReserve R{};
  const int64_t N = T * k;
  Carver c{base, 0};
  R.idx = static_cast<int32_t*>(c.take(N * 4));
  R.w = static_cast<float*>(c.take(N * 4));
  R.counts = static_cast<int32_t*>(c.take(E * 4));
  R.offsets = static_cast<int32_t*>(c.take((E + 1) * 4));
  R.perm = static_cast<int32_t*>(c.take(N * 4));
  R.slot_row = static_cast<int32_t*>(c.take(N * 4));
  R.dropped = static_cast<uint8_t*>(c.take(N));
  R.dws = c.take(dispatch_ws_bytes(T, E));
  R.fws = c.take(tiled_ws_bytes());
  R.g = c.take((size_t)N * F * 2);
  R.u = c.take((size_t)N * F * 2);
  R.h = c.take((size_t)(N + kBwdSlackRows) * F * 2);
  R.y = c.take((size_t)N * H * 2);
  R.total = c.off;
  return R;
}

// Backward scratch: the row-layout gradients and the gathered x rows.
struct BwdWs {
  void* dy;     // [N + slack][H]
  void* dh;     // [N][F]
  void* dgu;    // [N + slack][2F]: dg then du
  void* dxr;    // [N][H]
  void* xg;     // [N + slack][H]: x rows in dispatch order
  float* dw;    // [N]
  float* dl;    // [T][E]
  float* part;  // router gradient partials
  int32_t* cnt; // [1] rows per rank of the gather (one rank)
  void* tws;    // tile scratch of the data-gradient products
  size_t total;
};

BwdWs bwd_ws_layout(char* base, int64_t T, int32_t H, int32_t F, int32_t E, int32_t k) {
  BwdWs B{};
  const int64_t N = T * k, Ns = N + kBwdSlackRows;
  const size_t h = (size_t)H, f = (size_t)F;
  Carver c{base, 0};
  B.dy = c.take((size_t)Ns * h * 2);
  B.dh = c.take((size_t)N * f * 2);
  B.dgu = c.take((size_t)Ns * 2 * f * 2);
  B.dxr = c.take((size_t)N * h * 2);
  B.xg = c.take((size_t)Ns * h * 2);
  B.dw = static_cast<float*>(c.take((size_t)N * 4));
  B.dl = static_cast<float*>(c.take((size_t)T * E * 4));
  B.part = static_cast<float*>(c.take((size_t)router_wgrad_chunks(T) * E * h * 4));
  B.cnt = static_cast<int32_t*>(c.take(4));
  B.tws = c.take(tiled_ws_bytes());
  B.total = c.off;
  return B;
}

// Training: bf16 activations and weights; row indices (with the 64 slack
// rows) stay below 2^31.
moe_status check_train(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k, moe_dtype act,
                       moe_dtype wt) {
  moe_status st;
  if ((st = check_shape(T, E, k)) || (st = check_dim("H", H)) || (st = check_dim("F", F)))
    return st;
  REQUIRE(act == MOE_BF16 && wt == MOE_BF16, MOE_ERR_UNSUPPORTED,
          "training entry points support bf16 activations and weights only (got %d, %d)",
          (int)act, (int)wt);
  REQUIRE(T * (int64_t)k + kBwdSlackRows < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED,
          "training supports T*k < 2^31 - 64 (got %lld)", (long long)(T * k));
  return ok();
}

// Kernel choice: float32 -> VALU tiles; bf16 with T <= kDecodeMaxT (so at
// most kDecodeMaxT rows per expert) -> weight-streaming decode kernels;
// otherwise the MFMA grouped GEMM tiles.
hipError_t launch_gateup(const FfnArgs& a, moe_dtype act, moe_dtype wt, hipStream_t s) {
  if (act == MOE_F32) return launch_gateup_f32(a, s);
  if (a.T <= kDecodeMaxT) return launch_gateup_decode(a, (Wt)wt, s);
  return launch_gateup_tiled(a, (Wt)wt, s);
}

hipError_t launch_down(const FfnArgs& a, moe_dtype act, moe_dtype wt, hipStream_t s) {
  if (act == MOE_F32) return launch_down_f32(a, s);
  if (a.T <= kDecodeMaxT) return launch_down_decode(a, (Wt)wt, s);
  return launch_down_tiled(a, (Wt)wt, s);
}

moe_status run_ffn(const void* x, moe_dtype act, const int32_t* perm, const int32_t* offsets,
                   int64_t T, int32_t H, int32_t F, int32_t E, int32_t k, const void* wg,
                   const void* wu, const void* wd, moe_dtype wt, const float* sg, const float* su,
                   const float* sd, void* h, void* y, void* ws, hipStream_t s) {
  FfnArgs a{x, perm, offsets, T, H, F, E, k, wg, wu, wd, sg, su, sd, h, y, ws};
  hipError_t err = launch_gateup(a, act, wt, s);
  if (err != hipSuccess) return hip_status(err, "expert gate/up launch");
  return hip_status(launch_down(a, act, wt, s), "expert down launch");
}

moe_status check_ffn_common(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                            moe_dtype act, moe_dtype wt) {
  moe_status st;
  if ((st = check_shape(T, E, k)) || (st = check_dim("H", H)) || (st = check_dim("F", F)) ||
      (st = check_pair(act, wt)) || (st = check_int4(T, H, F, wt)))
    return st;
  return ok();
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_router_topk(const void* x, moe_dtype x_dtype, const float* w_router, int64_t T,
                           int32_t H, int32_t E, int32_t k, int32_t* topk_idx, float* topk_w,
                           float* logits, moe_stream_t stream) {
  moe_status st;
  if ((st = check_shape(T, E, k)) || (st = check_dim("H", H)) || (st = check_act(x_dtype)))
    return st;
  if (T == 0) return ok();  // T-sized buffers may be NULL
  REQUIRE(x && w_router && topk_idx && topk_w, MOE_ERR_INVALID_ARGUMENT,
          "x, w_router, topk_idx and topk_w must be non-NULL");
  REQUIRE(aligned16(x) && aligned16(w_router), MOE_ERR_INVALID_ARGUMENT,
          "x and w_router must be 16-byte aligned");
  return hip_status(launch_router_topk(x, x_dtype == MOE_F32 ? ACT_F32 : ACT_BF16, w_router, T, H,
                                       E, k, topk_idx, topk_w, logits, (hipStream_t)stream),
                    "router launch");
}

size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k) {
  (void)k;
  if (T < 0 || E < 1) return 0;
  return dispatch_ws_bytes(T, E);
}

moe_status moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t E, int32_t k,
                        float capacity_factor, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* slot_row, uint8_t* dropped, void* ws, size_t ws_bytes,
                        moe_stream_t stream) {
  moe_status st;
  if ((st = check_shape(T, E, k))) return st;
  REQUIRE(counts && offsets, MOE_ERR_INVALID_ARGUMENT, "counts and offsets must be non-NULL");
  REQUIRE(!std::isnan(capacity_factor), MOE_ERR_INVALID_ARGUMENT, "capacity_factor is NaN");
  if (T == 0) {
    // counts and offsets of an empty input are zeros; T-sized buffers may be NULL
    hipError_t e = launch_fill_i32(counts, E, 0, (hipStream_t)stream);
    if (e == hipSuccess) e = launch_fill_i32(offsets, E + 1, 0, (hipStream_t)stream);
    return hip_status(e, "dispatch (empty input)");
  }
  REQUIRE(topk_idx && perm && slot_row && dropped, MOE_ERR_INVALID_ARGUMENT,
          "topk_idx, perm, slot_row and dropped must be non-NULL");
  const size_t need = dispatch_ws_bytes(T, E);
  REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE_TOO_SMALL,
          "dispatch workspace: need %zu bytes, got %zu", need, ws ? ws_bytes : (size_t)0);
  const int64_t cap = capacity_of(T, k, E, capacity_factor);
  return hip_status(launch_dispatch(topk_idx, T, E, k, cap, counts, offsets, perm, slot_row,
                                    dropped, ws, (hipStream_t)stream),
                    "dispatch launch");
}

size_t moe_expert_ffn_workspace_bytes(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                                      moe_dtype act_dtype, moe_dtype w_dtype) {
  if (T < 0 || H < 1 || F < 1 || E < 1 || k < 1) return 0;
  return ffn_ws_bytes(T, H, F, E, k, act_dtype == MOE_F32 ? ACT_F32 : ACT_BF16, (Wt)w_dtype);
}

moe_status moe_expert_ffn(const void* x, moe_dtype act_dtype, const int32_t* perm,
                          const int32_t* offsets, int64_t T, int32_t H, int32_t F, int32_t E,
                          int32_t k, const void* w_gate, const void* w_up, const void* w_down,
                          moe_dtype w_dtype, const float* s_gate, const float* s_up,
                          const float* s_down, void* h, void* y_perm, void* ws, size_t ws_bytes,
                          moe_stream_t stream) {
  moe_status st;
  if ((st = check_shape(T, E, k)) || (st = check_dim("H", H)) || (st = check_dim("F", F)) ||
      (st = check_pair(act_dtype, w_dtype)) || (st = check_int4(T, H, F, w_dtype)))
    return st;
  if (T == 0) return ok();  // T-sized buffers may be NULL
  REQUIRE(x && perm && offsets && w_gate && w_up && w_down && h && y_perm,
          MOE_ERR_INVALID_ARGUMENT,
          "x, perm, offsets, w_gate, w_up, w_down, h and y_perm must be non-NULL");
  const bool i8 = has_scales(w_dtype);
  REQUIRE(i8 == (s_gate && s_up && s_down) && (i8 || (!s_gate && !s_up && !s_down)),
          MOE_ERR_INVALID_ARGUMENT,
          "scales must be given exactly when weights are MOE_I8 or MOE_I4");
  REQUIRE(aligned16(x) && aligned16(w_gate) && aligned16(w_up) && aligned16(w_down) &&
              aligned16(h) && aligned16(y_perm),
          MOE_ERR_INVALID_ARGUMENT, "x, weights, h and y_perm must be 16-byte aligned");
  const size_t need = ffn_ws_bytes(T, H, F, E, k, act_dtype == MOE_F32 ? ACT_F32 : ACT_BF16,
                                   (Wt)w_dtype);
  REQUIRE(ws_bytes >= need && (need == 0 || ws), MOE_ERR_WORKSPACE_TOO_SMALL,
          "expert FFN workspace: need %zu bytes, got %zu", need, ws_bytes);
  if (T == 0) return ok();
  return run_ffn(x, act_dtype, perm, offsets, T, H, F, E, k, w_gate, w_up, w_down, w_dtype,
                 s_gate, s_up, s_down, h, y_perm, ws, (hipStream_t)stream);
}

moe_status moe_expert_gate_up(const void* x, moe_dtype act_dtype, const int32_t* perm,
                              const int32_t* offsets, int64_t T, int32_t H, int32_t F, int32_t E,
                              int32_t k, const void* w_gate, const void* w_up, moe_dtype w_dtype,
                              const float* s_gate, const float* s_up, void* h,
                              moe_stream_t stream) {
  moe_status st;
  if ((st = check_ffn_common(T, H, F, E, k, act_dtype, w_dtype))) return st;
  if (T == 0) return ok();  // T-sized buffers may be NULL
  REQUIRE(x && perm && offsets && w_gate && w_up && h, MOE_ERR_INVALID_ARGUMENT,
          "x, perm, offsets, w_gate, w_up and h must be non-NULL");
  const bool i8 = has_scales(w_dtype);
  REQUIRE(i8 == (s_gate && s_up) && (i8 || (!s_gate && !s_up)), MOE_ERR_INVALID_ARGUMENT,
          "scales must be given exactly when weights are MOE_I8 or MOE_I4");
  REQUIRE(aligned16(x) && aligned16(w_gate) && aligned16(w_up) && aligned16(h),
          MOE_ERR_INVALID_ARGUMENT, "x, weights and h must be 16-byte aligned");
  FfnArgs a{x, perm, offsets, T, H, F, E, k, w_gate, w_up, nullptr, s_gate, s_up, nullptr, h,
            nullptr, nullptr};
  return hip_status(launch_gateup(a, act_dtype, w_dtype, (hipStream_t)stream),
                    "expert gate/up launch");
}

moe_status moe_expert_down(const void* h, moe_dtype act_dtype, const int32_t* offsets, int64_t T,
                           int32_t H, int32_t F, int32_t E, int32_t k, const void* w_down,
                           moe_dtype w_dtype, const float* s_down, void* y_perm, void* ws,
                           size_t ws_bytes, moe_stream_t stream) {
  moe_status st;
  if ((st = check_ffn_common(T, H, F, E, k, act_dtype, w_dtype))) return st;
  if (T == 0) return ok();  // T-sized buffers may be NULL
  REQUIRE(h && offsets && w_down && y_perm, MOE_ERR_INVALID_ARGUMENT,
          "h, offsets, w_down and y_perm must be non-NULL");
  REQUIRE(has_scales(w_dtype) == (s_down != nullptr), MOE_ERR_INVALID_ARGUMENT,
          "s_down must be given exactly when weights are MOE_I8 or MOE_I4");
  REQUIRE(aligned16(h) && aligned16(w_down) && aligned16(y_perm), MOE_ERR_INVALID_ARGUMENT,
          "h, w_down and y_perm must be 16-byte aligned");
  const size_t need = ffn_ws_bytes(T, H, F, E, k, act_dtype == MOE_F32 ? ACT_F32 : ACT_BF16,
                                   (Wt)w_dtype);
  REQUIRE(ws_bytes >= need && (need == 0 || ws), MOE_ERR_WORKSPACE_TOO_SMALL,
          "expert down workspace: need %zu bytes, got %zu", need, ws_bytes);
  if (T == 0) return ok();
  FfnArgs a{nullptr, nullptr, offsets, T, H, F, E, k, nullptr, nullptr, w_down, nullptr, nullptr,
            s_down, const_cast<void*>(h), y_perm, ws};
  return hip_status(launch_down(a, act_dtype, w_dtype, (hipStream_t)stream),
                    "expert down launch");
}

moe_status moe_combine(const void* y_perm, const int32_t* slot_row, const float* topk_w,
                       int64_t T, int32_t H, int32_t k, moe_dtype act_dtype, void* out,
                       moe_stream_t stream) {
  moe_status st;
  REQUIRE(T >= 0, MOE_ERR_INVALID_ARGUMENT, "T must be >= 0");
  REQUIRE(k >= 1, MOE_ERR_INVALID_ARGUMENT, "k must be >= 1");
  REQUIRE(k <= 4, MOE_ERR_UNSUPPORTED, "k=%d > 4 is not supported", k);
  if ((st = check_dim("H", H)) || (st = check_act(act_dtype))) return st;
  if (T == 0) return ok();  // T-sized buffers may be NULL
  REQUIRE(y_perm && slot_row && topk_w && out, MOE_ERR_INVALID_ARGUMENT,
          "y_perm, slot_row, topk_w and out must be non-NULL");
  REQUIRE(aligned16(y_perm) && aligned16(out), MOE_ERR_INVALID_ARGUMENT,
          "y_perm and out must be 16-byte aligned");
  return hip_status(launch_combine(y_perm, slot_row, topk_w, T, H, k,
                                   act_dtype == MOE_F32 ? ACT_F32 : ACT_BF16, out,
                                   (hipStream_t)stream),
                    "combine launch");
}

moe_status moe_routing_stats(const float* logits, const int32_t* counts, int64_t T, int32_t E,
                             int32_t k, float* utilization, float* margin,
                             float* unselected_mass, moe_stream_t stream) {
  moe_status st;
  if ((st = check_shape(T, E, k))) return st;
  const bool per_token = (margin || unselected_mass) && T > 0;
  if (!utilization && !per_token) return ok();
  REQUIRE(!utilization || counts, MOE_ERR_INVALID_ARGUMENT,
          "counts must be non-NULL when utilization is requested");
  REQUIRE(!per_token || logits, MOE_ERR_INVALID_ARGUMENT,
          "logits must be non-NULL when margin or unselected_mass is requested");
  return hip_status(launch_routing_stats(logits, counts, T, E, k, utilization,
                                         per_token ? margin : nullptr,
                                         per_token ? unselected_mass : nullptr,
                                         (hipStream_t)stream),
                    "routing statistics launch");
}

moe_status moe_ep_pack(const void* x, moe_dtype act_dtype, const int32_t* perm,
                       const int32_t* offsets, int64_t T, int32_t H, int32_t E, int32_t k,
                       int32_t R, void* send_buf, int32_t* send_counts, moe_stream_t stream) {
  moe_status st;
  if ((st = check_shape(T, E, k)) || (st = check_dim("H", H)) || (st = check_act(act_dtype)))
    return st;
  REQUIRE(R >= 1 && R <= 64, MOE_ERR_UNSUPPORTED, "R=%d ranks: 1 <= R <= 64 supported", R);
  REQUIRE(E % R == 0, MOE_ERR_INVALID_ARGUMENT, "E=%d is not a multiple of R=%d", E, R);
  REQUIRE(offsets && send_counts, MOE_ERR_INVALID_ARGUMENT,
          "offsets and send_counts must be non-NULL");
  if (T > 0) {
    REQUIRE(x && perm && send_buf, MOE_ERR_INVALID_ARGUMENT,
            "x, perm and send_buf must be non-NULL");
    REQUIRE(aligned16(x) && aligned16(send_buf), MOE_ERR_INVALID_ARGUMENT,
            "x and send_buf must be 16-byte aligned");
  }
  return hip_status(launch_ep_pack(x, (int64_t)H * act_size(act_dtype), perm, offsets, T * k, E,
                                   k, R, send_buf, send_counts, (hipStream_t)stream),
                    "EP pack launch");
}

moe_status moe_ep_recv_layout(const int32_t* recv_counts, int32_t R, int32_t E_local,
                              int64_t max_rows, int32_t* local_offsets, int32_t* row_index,
                              moe_stream_t stream) {
  REQUIRE(R >= 1 && R <= 64, MOE_ERR_UNSUPPORTED, "R=%d ranks: 1 <= R <= 64 supported", R);
  REQUIRE(E_local >= 1 && E_local <= 16, MOE_ERR_UNSUPPORTED,
          "E_local=%d: 1 <= E_local <= 16 supported", E_local);
  REQUIRE(max_rows >= 0 && max_rows < ((int64_t)1 << 31), MOE_ERR_INVALID_ARGUMENT,
          "max_rows=%lld must be in [0, 2^31)", (long long)max_rows);
  REQUIRE(recv_counts && local_offsets && (row_index || max_rows == 0),
          MOE_ERR_INVALID_ARGUMENT,
          "recv_counts, local_offsets and row_index (unless max_rows == 0) must be non-NULL");
  return hip_status(launch_ep_recv_layout(recv_counts, R, E_local, max_rows, local_offsets,
                                          row_index, (hipStream_t)stream),
                    "EP receive layout launch");
}

moe_status moe_ep_unpack(const void* y_rows, moe_dtype act_dtype, const int32_t* row_index,
                         const int32_t* local_offsets, int32_t E_local, int32_t H,
                         int64_t max_rows, void* back_buf, moe_stream_t stream) {
  moe_status st;
  if ((st = check_dim("H", H)) || (st = check_act(act_dtype))) return st;
  REQUIRE(E_local >= 1 && E_local <= 16, MOE_ERR_UNSUPPORTED,
          "E_local=%d: 1 <= E_local <= 16 supported", E_local);
  REQUIRE(max_rows >= 0 && max_rows < ((int64_t)1 << 31), MOE_ERR_INVALID_ARGUMENT,
          "max_rows=%lld must be in [0, 2^31)", (long long)max_rows);
  if (max_rows == 0) return ok();
  REQUIRE(y_rows && row_index && local_offsets && back_buf, MOE_ERR_INVALID_ARGUMENT,
          "y_rows, row_index, local_offsets and back_buf must be non-NULL");
  REQUIRE(aligned16(y_rows) && aligned16(back_buf), MOE_ERR_INVALID_ARGUMENT,
          "y_rows and back_buf must be 16-byte aligned");
  return hip_status(launch_ep_unpack(y_rows, (int64_t)H * act_size(act_dtype), row_index,
                                     local_offsets, E_local, max_rows, back_buf,
                                     (hipStream_t)stream),
                    "EP unpack launch");
}

size_t moe_layer_workspace_bytes(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                                 moe_dtype act_dtype, moe_dtype w_dtype) {
  if (T < 0 || H < 1 || F < 1 || E < 1 || k < 1) return 0;
  return layer_ws_layout(nullptr, T, H, F, E, k, act_dtype, w_dtype).total;
}

}  // extern "C"

namespace {

// The layer forward's argument checks (everything but the workspace).
moe_status check_layer(const void* x, moe_dtype act_dtype, const float* w_router,
                       const void* w_gate, const void* w_up, const void* w_down,
                       moe_dtype w_dtype, const float* s_gate, const float* s_up,
                       const float* s_down, int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                       float capacity_factor, const void* out) {
  moe_status st;
  if ((st = check_shape(T, E, k)) || (st = check_dim("H", H)) || (st = check_dim("F", F)) ||
      (st = check_pair(act_dtype, w_dtype)) || (st = check_int4(T, H, F, w_dtype)))
    return st;
  REQUIRE(!std::isnan(capacity_factor), MOE_ERR_INVALID_ARGUMENT, "capacity_factor is NaN");
  if (T == 0) return ok();
  REQUIRE(x && w_router && w_gate && w_up && w_down && out, MOE_ERR_INVALID_ARGUMENT,
          "x, w_router, w_gate, w_up, w_down and out must be non-NULL");
  const bool i8 = has_scales(w_dtype);
  REQUIRE(i8 == (s_gate && s_up && s_down) && (i8 || (!s_gate && !s_up && !s_down)),
          MOE_ERR_INVALID_ARGUMENT,
          "scales must be given exactly when weights are MOE_I8 or MOE_I4");
  REQUIRE(aligned16(x) && aligned16(w_router) && aligned16(w_gate) && aligned16(w_up) &&
              aligned16(w_down) && aligned16(out),
          MOE_ERR_INVALID_ARGUMENT, "x, weights and out must be 16-byte aligned");
  return ok();
}

// The layer forward's launches, on a checked workspace of the layer's size.
moe_status run_layer(const void* x, moe_dtype act_dtype, const float* w_router,
                     const void* w_gate, const void* w_up, const void* w_down, moe_dtype w_dtype,
                     const float* s_gate, const float* s_up, const float* s_down, int64_t T,
                     int32_t H, int32_t F, int32_t E, int32_t k, float capacity_factor, void* out,
                     int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                     uint8_t* dropped, void* ws, moe_stream_t stream) {
  moe_status st;
  if (T == 0) {
    // nothing to compute; the optional per-expert outputs are zeros
    hipError_t e = hipSuccess;
    if (counts) e = launch_fill_i32(counts, E, 0, (hipStream_t)stream);
    if (e == hipSuccess && offsets) e = launch_fill_i32(offsets, E + 1, 0, (hipStream_t)stream);
    return hip_status(e, "layer (empty input)");
  }
  hipStream_t s = (hipStream_t)stream;
  LayerWs L = layer_ws_layout(static_cast<char*>(ws), T, H, F, E, k, act_dtype, w_dtype);
  int32_t* idx = topk_idx ? topk_idx : L.idx;
  float* w = topk_w ? topk_w : L.w;
  int32_t* cnt = counts ? counts : L.counts;
  int32_t* off = offsets ? offsets : L.offsets;
  uint8_t* drp = dropped ? dropped : L.dropped;
  const Act act = act_dtype == MOE_F32 ? ACT_F32 : ACT_BF16;
  hipError_t e = launch_router_topk(x, act, w_router, T, H, E, k, idx, w, nullptr, s);
  if (e != hipSuccess) return hip_status(e, "router launch");
  const int64_t cap = capacity_of(T, k, E, capacity_factor);
  e = launch_dispatch(idx, T, E, k, cap, cnt, off, L.perm, L.slot_row, drp, L.dws, s);
  if (e != hipSuccess) return hip_status(e, "dispatch launch");
  st = run_ffn(x, act_dtype, L.perm, off, T, H, F, E, k, w_gate, w_up, w_down, w_dtype, s_gate,
               s_up, s_down, L.h, L.y, L.fws, s);
  if (st) return st;
  return hip_status(launch_combine(L.y, L.slot_row, w, T, H, k, act, out, s), "combine launch");
}

}  // namespace

extern "C" {

moe_status moe_layer_forward(const void* x, moe_dtype act_dtype, const float* w_router,
                             const void* w_gate, const void* w_up, const void* w_down,
                             moe_dtype w_dtype, const float* s_gate, const float* s_up,
                             const float* s_down, int64_t T, int32_t H, int32_t F, int32_t E,
                             int32_t k, float capacity_factor, void* out, int32_t* topk_idx,
                             float* topk_w, int32_t* counts, int32_t* offsets, uint8_t* dropped,
                             void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status st;
  if ((st = check_layer(x, act_dtype, w_router, w_gate, w_up, w_down, w_dtype, s_gate, s_up,
                        s_down, T, H, F, E, k, capacity_factor, out)))
    return st;
  if (T > 0) {
    const size_t need = layer_ws_layout(nullptr, T, H, F, E, k, act_dtype, w_dtype).total;
    REQUIRE(ws && ws_bytes >= need && aligned16(ws), MOE_ERR_WORKSPACE_TOO_SMALL,
            "layer workspace: need %zu bytes (16-byte aligned), got %zu", need,
            ws ? ws_bytes : (size_t)0);
  }
  return run_layer(x, act_dtype, w_router, w_gate, w_up, w_down, w_dtype, s_gate, s_up, s_down,
                   T, H, F, E, k, capacity_factor, out, topk_idx, topk_w, counts, offsets,
                   dropped, ws, stream);
}

moe_status moe_layer_forward_noalloc(const void* x, moe_dtype act_dtype, const float* w_router,
                                     const void* w_gate, const void* w_up, const void* w_down,
                                     moe_dtype w_dtype, const float* s_gate, const float* s_up,
                                     const float* s_down, int64_t T, int32_t H, int32_t F,
                                     int32_t E, int32_t k, float capacity_factor, void* out,
                                     int32_t* topk_idx, float* topk_w, int32_t* counts,
                                     int32_t* offsets, uint8_t* dropped, moe_stream_t stream) {
  moe_status st;
  if ((st = check_layer(x, act_dtype, w_router, w_gate, w_up, w_down, w_dtype, s_gate, s_up,
                        s_down, T, H, F, E, k, capacity_factor, out)))
    return st;
  void* ws = nullptr;
  if (T > 0) {
    const size_t need = layer_ws_layout(nullptr, T, H, F, E, k, act_dtype, w_dtype).total;
    REQUIRE(need <= MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_UNSUPPORTED,
            "moe_layer_forward_noalloc: this shape needs %zu bytes of workspace, above the "
            "library's fixed %zu (use moe_layer_forward with a workspace)",
            need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    const hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "moe_layer_forward_noalloc: scratch lookup");
  }
  return run_layer(x, act_dtype, w_router, w_gate, w_up, w_down, w_dtype, s_gate, s_up, s_down,
                   T, H, F, E, k, capacity_factor, out, topk_idx, topk_w, counts, offsets,
                   dropped, ws, stream);
}

size_t moe_layer_train_reserve_bytes(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k) {
  if (T < 0 || H < 1 || F < 1 || E < 1 || k < 1) return 0;
  return train_reserve_layout(nullptr, T, H, F, E, k).total;
}

size_t moe_layer_backward_workspace_bytes(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k) {
  if (T < 0 || H < 1 || F < 1 || E < 1 || k < 1) return 0;
  return bwd_ws_layout(nullptr, T, H, F, E, k).total;
}

moe_status moe_layer_forward_train(const void* x, moe_dtype act_dtype, const float* w_router,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   moe_dtype w_dtype, int64_t T, int32_t H, int32_t F, int32_t E,
                                   int32_t k, float capacity_factor, void* out, void* reserve,
                                   size_t reserve_bytes, moe_stream_t stream) {
  moe_status st;
  if ((st = check_train(T, H, F, E, k, act_dtype, w_dtype))) return st;
  REQUIRE(!std::isnan(capacity_factor), MOE_ERR_INVALID_ARGUMENT, "capacity_factor is NaN");
  const TrainReserve need = train_reserve_layout(nullptr, T, H, F, E, k);
  REQUIRE(reserve && reserve_bytes >= need.total && aligned16(reserve),
          MOE_ERR_WORKSPACE_TOO_SMALL,
          "training reserve: need %zu bytes (16-byte aligned), got %zu", need.total,
          reserve ? reserve_bytes : (size_t)0);
  hipStream_t s = (hipStream_t)stream;
  TrainReserve R = train_reserve_layout(static_cast<char*>(reserve), T, H, F, E, k);
  if (T == 0) {
    hipError_t e = launch_fill_i32(R.counts, E, 0, s);
    if (e == hipSuccess) e = launch_fill_i32(R.offsets, E + 1, 0, s);
    return hip_status(e, "training forward (empty input)");
  }
  REQUIRE(x && w_router && w_gate && w_up && w_down && out, MOE_ERR_INVALID_ARGUMENT,
          "x, w_router, w_gate, w_up, w_down and out must be non-NULL");
  REQUIRE(aligned16(x) && aligned16(w_router) && aligned16(w_gate) && aligned16(w_up) &&
              aligned16(w_down) && aligned16(out),
          MOE_ERR_INVALID_ARGUMENT, "x, weights and out must be 16-byte aligned");
  hipError_t e = launch_router_topk(x, ACT_BF16, w_router, T, H, E, k, R.idx, R.w, nullptr, s);
  if (e != hipSuccess) return hip_status(e, "router launch");
  const int64_t cap = capacity_of(T, k, E, capacity_factor);
  e = launch_dispatch(R.idx, T, E, k, cap, R.counts, R.offsets, R.perm, R.slot_row, R.dropped,
                      R.dws, s);
  if (e != hipSuccess) return hip_status(e, "dispatch launch");
  // the MFMA tiles at every T (the decode kernels keep no pre-activations)
  FfnArgs a{x, R.perm, R.offsets, T, H, F, E, k, w_gate, w_up, w_down, nullptr, nullptr, nullptr,
            R.h, R.y, R.fws, R.g, R.u};
  e = launch_gateup_save_tiled(a, s);
  if (e != hipSuccess) return hip_status(e, "expert gate/up launch");
  e = launch_down_tiled(a, WT_BF16, s);
  if (e != hipSuccess) return hip_status(e, "expert down launch");
  return hip_status(launch_combine(R.y, R.slot_row, R.w, T, H, k, ACT_BF16, out, s),
                    "combine launch");
}

}  // extern "C"

namespace {

// Checks shared by the backward entry points. data: dout and dx are needed
// (the data step); the weight gradients are checked by whichever step writes
// them.
moe_status check_backward(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k, moe_dtype act,
                          moe_dtype wt, const void* reserve, size_t reserve_bytes, const void* ws,
                          size_t ws_bytes) {
  moe_status st;
  if ((st = check_train(T, H, F, E, k, act, wt))) return st;
  const TrainReserve rneed = train_reserve_layout(nullptr, T, H, F, E, k);
  REQUIRE(reserve && reserve_bytes >= rneed.total && aligned16(reserve),
          MOE_ERR_WORKSPACE_TOO_SMALL, "training reserve: need %zu bytes, got %zu", rneed.total,
          reserve ? reserve_bytes : (size_t)0);
  const BwdWs wneed = bwd_ws_layout(nullptr, T, H, F, E, k);
  REQUIRE(ws && ws_bytes >= wneed.total && aligned16(ws), MOE_ERR_WORKSPACE_TOO_SMALL,
          "backward workspace: need %zu bytes (16-byte aligned), got %zu", wneed.total,
          ws ? ws_bytes : (size_t)0);
  return ok();
}

#define MOE_STEP(call, what)                          \
  do {                                                \
    hipError_t e_ = (call);                           \
    if (e_ != hipSuccess) return hip_status(e_, what); \
  } while (0)

// combine backward, dh = dy W_down, SwiGLU backward, dx rows = dg W_gate +
// du W_up, dx and the router gradient, all on the weights as stored; then the
// x rows in dispatch order for the weight step
moe_status backward_data(const void* x, const float* w_router, const void* w_gate,
                         const void* w_up, const void* w_down, int64_t T, int32_t H, int32_t F,
                         int32_t E, int32_t k, const void* dout, const TrainReserve& R,
                         void* dx, float* dw_router, const BwdWs& B, hipStream_t s) {
  const int64_t N = T * k;
  if (T > 0) {
    MOE_STEP(launch_combine_bwd(dout, R.y, R.slot_row, R.w, R.idx, T, H, E, k, B.dy, B.dw, B.dl,
                                s), "combine backward launch");
    const DgradArgs dh{B.dy, R.offsets, T, E, k, F, H, H, w_down, nullptr, B.dh, B.tws};
    MOE_STEP(launch_dgrad_nn(dh, s), "dh GEMM launch");
    MOE_STEP(launch_swiglu_bwd(B.dh, R.g, R.u, R.offsets, E, N, F, B.dgu, s),
             "SwiGLU backward launch");
    const DgradArgs dxr{B.dgu, R.offsets, T, E, k, H, 2 * F, F, w_gate, w_up, B.dxr, B.tws};
    MOE_STEP(launch_dgrad_nn(dxr, s), "dx GEMM launch");
    MOE_STEP(launch_dx_combine(B.dxr, R.slot_row, R.idx, B.dl, w_router, T, H, E, k, dx, s),
             "dx combine launch");
    MOE_STEP(launch_ep_pack(x, (int64_t)H * 2, R.perm, R.offsets, N, E, k, 1, B.xg, B.cnt, s),
             "x gather launch");
  }
  MOE_STEP(launch_router_wgrad(x, B.dl, T, H, E, B.part, dw_router, s), "router gradient launch");
  return ok();
}

// the weight gradients: per-expert contractions over the expert's rows
moe_status backward_weights(int32_t H, int32_t F, int32_t E, const TrainReserve& R,
                            void* dw_gate, void* dw_up, void* dw_down, const BwdWs& B,
                            hipStream_t s) {
  // dW_down[e] = dy_e^T h_e (M = H, N = F); the F-column operand is the
  // larger, so the m tiles that share one of its blocks run together
  const WgradTnArgs gd{B.dy, H, R.h, F, R.offsets, E, H, F, H, dw_down, nullptr, 1};
  MOE_STEP(launch_wgrad_tn(gd, s), "down weight gradient launch");
  // [dW_gate; dW_up][e] = [dg | du]_e^T x_e (M = 2F, N = H)
  const WgradTnArgs ggu{B.dgu, 2 * (int64_t)F, B.xg, H, R.offsets, E, 2 * F, H, F, dw_gate, dw_up,
                        0};
  MOE_STEP(launch_wgrad_tn(ggu, s), "gate/up weight gradient launch");
  return ok();
}
#undef MOE_STEP

}  // namespace

extern "C" {

moe_status moe_layer_backward_data(const void* x, moe_dtype act_dtype, const float* w_router,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   moe_dtype w_dtype, int64_t T, int32_t H, int32_t F, int32_t E,
                                   int32_t k, const void* dout, const void* reserve,
                                   size_t reserve_bytes, void* dx, float* dw_router, void* ws,
                                   size_t ws_bytes, moe_stream_t stream) {
  moe_status st;
  if ((st = check_backward(T, H, F, E, k, act_dtype, w_dtype, reserve, reserve_bytes, ws,
                           ws_bytes)))
    return st;
  REQUIRE(w_router && w_gate && w_up && w_down && dw_router, MOE_ERR_INVALID_ARGUMENT,
          "weights and dw_router must be non-NULL");
  REQUIRE(aligned16(w_router) && aligned16(w_gate) && aligned16(w_up) && aligned16(w_down) &&
              aligned16(dw_router),
          MOE_ERR_INVALID_ARGUMENT, "weights and dw_router must be 16-byte aligned");
  if (T > 0) {
    REQUIRE(x && dout && dx, MOE_ERR_INVALID_ARGUMENT, "x, dout and dx must be non-NULL");
    REQUIRE(aligned16(x) && aligned16(dout) && aligned16(dx), MOE_ERR_INVALID_ARGUMENT,
            "x, dout and dx must be 16-byte aligned");
  }
  const TrainReserve R =
      train_reserve_layout(static_cast<char*>(const_cast<void*>(reserve)), T, H, F, E, k);
  const BwdWs B = bwd_ws_layout(static_cast<char*>(ws), T, H, F, E, k);
  return backward_data(x, w_router, w_gate, w_up, w_down, T, H, F, E, k, dout, R, dx, dw_router,
                       B, (hipStream_t)stream);
}

moe_status moe_layer_backward_weights(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                                      const void* reserve, size_t reserve_bytes, void* dw_gate,
                                      void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                                      moe_stream_t stream) {
  moe_status st;
  if ((st = check_backward(T, H, F, E, k, MOE_BF16, MOE_BF16, reserve, reserve_bytes, ws,
                           ws_bytes)))
    return st;
  REQUIRE(dw_gate && dw_up && dw_down, MOE_ERR_INVALID_ARGUMENT,
          "dw_gate, dw_up and dw_down must be non-NULL");
  REQUIRE(aligned16(dw_gate) && aligned16(dw_up) && aligned16(dw_down), MOE_ERR_INVALID_ARGUMENT,
          "dw_gate, dw_up and dw_down must be 16-byte aligned");
  const TrainReserve R =
      train_reserve_layout(static_cast<char*>(const_cast<void*>(reserve)), T, H, F, E, k);
  const BwdWs B = bwd_ws_layout(static_cast<char*>(ws), T, H, F, E, k);
  return backward_weights(H, F, E, R, dw_gate, dw_up, dw_down, B, (hipStream_t)stream);
}

moe_status moe_layer_backward(const void* x, moe_dtype act_dtype, const float* w_router,
                              const void* w_gate, const void* w_up, const void* w_down,
                              moe_dtype w_dtype, int64_t T, int32_t H, int32_t F, int32_t E,
                              int32_t k, const void* dout, const void* reserve,
                              size_t reserve_bytes, void* dx, float* dw_router, void* dw_gate,
                              void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                              moe_stream_t stream) {
  moe_status st;
  // the weight step's own checks first, so that a failure enqueues nothing
  REQUIRE(dw_gate && dw_up && dw_down, MOE_ERR_INVALID_ARGUMENT,
          "dw_gate, dw_up and dw_down must be non-NULL");
  REQUIRE(aligned16(dw_gate) && aligned16(dw_up) && aligned16(dw_down), MOE_ERR_INVALID_ARGUMENT,
          "dw_gate, dw_up and dw_down must be 16-byte aligned");
  if ((st = moe_layer_backward_data(x, act_dtype, w_router, w_gate, w_up, w_down, w_dtype, T, H,
                                    F, E, k, dout, reserve, reserve_bytes, dx, dw_router, ws,
                                    ws_bytes, stream)))
    return st;
  return moe_layer_backward_weights(T, H, F, E, k, reserve, reserve_bytes, dw_gate, dw_up,
                                    dw_down, ws, ws_bytes, stream);
}

}  // extern "C"
