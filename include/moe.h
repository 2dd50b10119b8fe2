/*
 * moe.h -- C ABI of the top-2 mixture-of-experts FFN layer for AMD MI355X (gfx950).
 *
 * The layer is the one described on the n4n.ai page "How does Grok-1 use a
 * mixture-of-experts design?":
 *   - a bias-free router linear from the hidden size to E expert logits
 *     (section "The high-level architecture", GrokMoELayer; section
 *     "Routing: top-2 without auxiliary loss", grok_router_forward);
 *   - the top-k experts per token (k = 2 on the page) with a softmax taken
 *     over only the k selected logits (same sections);
 *   - dispatch of tokens to experts, with capacity-aware dropping when a
 *     finite capacity factor is given (grok_router_forward and the paragraph
 *     after it: capacity factor 1.25, overflow dropped in training, no drop at
 *     inference);
 *   - E independent SwiGLU experts w_down(silu(w_gate x) * w_up x) (section
 *     "Expert implementation: SwiGLU at scale"; gate and up may be fused into
 *     one product, FusedSwiGLUExpert);
 *   - the weighted combine of each token's expert outputs back to token order
 *     (GrokMoELayer.forward and the expert-parallel pseudocode in "Expert
 *     parallelism vs. tensor parallelism", which scales each expert output by
 *     its routing weight and skips experts that received no tokens).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA storage),
 *     row-major, contiguous, owned by the caller. The library allocates and
 *     frees nothing and keeps no state between calls apart from cached device
 *     properties; concurrent calls on different streams are safe as long as
 *     they do not share output or workspace buffers.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *     enqueues kernels on it and returns; nothing synchronises the stream,
 *     and no call copies data between host and device.
 *   - Shapes: T tokens (flattened batch*seq), H hidden, F expert dim, E
 *     experts, k experts per token. Supported: T >= 0, T*k < 2^31,
 *     1 <= E <= 16, 1 <= k <= min(E, 4), 64 <= H, F <= 2^20 with
 *     H % 64 == 0 and F % 64 == 0.
 *   - dtypes: activations (x, h, y_perm, out) are MOE_F32 or MOE_BF16; expert
 *     weights are MOE_F32 (with f32 activations), MOE_BF16, MOE_I8 or MOE_I4
 *     (with bf16 activations). The router weight, routing weights and scales
 *     are always float32; indices are int32.
 *   - Weights follow nn.Linear's [out, in] layout: w_gate, w_up are [E][F][H],
 *     w_down is [E][H][F], the router weight is [E][H]. int8 weights carry one
 *     float32 scale per output row (s_gate, s_up [E][F], s_down [E][H]); the
 *     effective weight is q * s.
 *   - MOE_I4 (page: 4-bit weights in sections "Inference: the real
 *     engineering challenge" and "Tradeoffs: when MoE wins and when it
 *     doesn't", AWQ/GPTQ named, no scheme given): each weight row of K
 *     values is K/2 bytes, byte j holding k = 2j in its low nibble and
 *     k = 2j+1 in its high nibble; a nibble is a code u in 0..15 meaning
 *     u - 8. One float32 scale per row and group of 128 consecutive k:
 *     s_gate, s_up [E][F][H/128], s_down [E][H][F/128]; the effective weight
 *     is (u - 8) * s. Supported for T <= 16 (the decode kernels) with H and F
 *     multiples of 128 and one expert's codes under 2 GiB (H*F/2 < 2^31);
 *     otherwise MOE_ERR_UNSUPPORTED.
 *   - Errors: every argument is checked before any HIP call; a failed check
 *     returns a non-zero status and enqueues nothing. A failed kernel launch
 *     returns MOE_ERR_HIP. moe_last_error() gives a message for the last
 *     failure on the calling thread. Nothing throws across the ABI.
 *   - T == 0 is valid and returns MOE_OK; buffers whose size scales with T
 *     may then be NULL. moe_dispatch and moe_layer_forward still write zeros
 *     to counts/offsets (when given); nothing else is launched.
 *   - Results are deterministic: no floating-point atomics, fixed reduction
 *     orders; two calls with the same inputs give bitwise-equal outputs.
 *   - NaN / Inf inputs are outside the contract.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, k > E, ... */
  MOE_ERR_UNSUPPORTED = 2,        /* valid but unsupported shape / dtype combination */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_I8 = 2, MOE_I4 = 3 } moe_dtype;

typedef void* moe_stream_t;       /* hipStream_t */

/* Name of a status code (static string). */
const char* moe_status_string(moe_status s);

/* Message describing the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------------------
 * Router + top-k + softmax (one fused kernel).
 * Page: "Routing: top-2 without auxiliary loss" (grok_router_forward) and
 * GrokMoELayer.forward in "The high-level architecture".
 *
 *   logits[t,e] = sum_h x[t,h] * w_router[e,h]      (float32 accumulation)
 *   topk_idx[t,0..k-1]: the k largest logits in descending order; equal
 *       logits rank the lower expert index first
 *   topk_w[t,j] = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0)
 *
 * x        [T,H]  MOE_F32 or MOE_BF16 (x_dtype)
 * w_router [E,H]  float32
 * topk_idx [T,k]  int32 (out); topk_w [T,k] float32 (out)
 * logits   [T,E]  float32 (out, optional: may be NULL)
 * ------------------------------------------------------------------------ */
moe_status moe_router_topk(const void* x, moe_dtype x_dtype, const float* w_router,
                           int64_t T, int32_t H, int32_t E, int32_t k,
                           int32_t* topk_idx, float* topk_w, float* logits,
                           moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Dispatch: group the T*k assignments a = t*k + j by expert, in token order,
 * and drop assignments over capacity.
 * Page: grok_router_forward (one-hot dispatch mask, capacity-aware dropping
 * when the factor is finite) and the paragraph after it (capacity factor x
 * mean load per expert; no dropping at inference).
 *
 *   cap = ceil(capacity_factor * (T*k) / E), evaluated in double precision;
 *         no limit when capacity_factor <= 0 or is infinite
 *   rank(t,j) = number of tokens t' < t that chose expert idx[t,j]
 *   kept(t,j) = rank(t,j) < cap
 *   counts[e]  = number of assignments to e (before the drop)      [E]
 *   offsets[e] = sum_{e'<e} min(counts[e'], cap); offsets[E] = kept total [E+1]
 *   perm[offsets[e] + rank] = t*k + j for kept assignments; the tail
 *                perm[offsets[E] .. T*k-1] is set to -1                   [T*k]
 *   slot_row[t*k+j] = offsets[e] + rank if kept, else -1                  [T*k]
 *   dropped[t*k+j]  = 1 if not kept, else 0                      uint8    [T*k]
 *
 * topk_idx [T,k] int32 with entries in [0,E) and distinct per token (the
 * router's output); out-of-range entries give undefined results.
 * ws: device scratch of at least moe_dispatch_workspace_bytes(T,E,k) bytes.
 * ------------------------------------------------------------------------ */
size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k);
moe_status moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t E, int32_t k,
                        float capacity_factor, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* slot_row, uint8_t* dropped,
                        void* ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Expert FFN over the dispatched rows (all experts, one call).
 * Page: "Expert implementation: SwiGLU at scale" (SwiGLUExpert and the fused
 * gate/up form, FusedSwiGLUExpert).
 *
 * For every expert e and row r in [offsets[e], offsets[e+1]), with token
 * t = perm[r] / k:
 *   h[r,:]      = silu(x[t,:] W_gate[e]^T) * (x[t,:] W_up[e]^T)        [T*k, F]
 *   y_perm[r,:] = h[r,:] W_down[e]^T                                 [T*k, H]
 * silu(g) = g / (1 + exp(-g)). Products accumulate in float32; with bf16
 * activations h is rounded to bf16 once (after silu(g)*u) and y_perm once.
 * int8 weights are converted exactly to bf16 and each output column of the
 * float32 accumulator is multiplied by its row scale; int4 codes are
 * converted exactly and each 128-k group's partial sum is multiplied by its
 * scale.
 * Rows at or past offsets[E] of h and y_perm are left unwritten.
 *
 * x [T,H] (act_dtype); perm [T*k] and offsets [E+1] from moe_dispatch;
 * h [T*k,F] and y_perm [T*k,H] (act_dtype, out);
 * s_gate/s_up/s_down must be non-NULL exactly when w_dtype is MOE_I8 or
 * MOE_I4. Supported (act, weight) pairs: (F32,F32), (BF16,BF16), (BF16,I8),
 * (BF16,I4).
 * ws: device scratch of at least moe_expert_ffn_workspace_bytes(...) bytes
 * (may be 0, then ws may be NULL; with bf16 activations it is the decode
 * path's split-k partials for T <= 16, else 192 MiB for the float32
 * partials of the down projection's split tail tiles).
 * ------------------------------------------------------------------------ */
size_t moe_expert_ffn_workspace_bytes(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                                      moe_dtype act_dtype, moe_dtype w_dtype);
moe_status moe_expert_ffn(const void* x, moe_dtype act_dtype,
                          const int32_t* perm, const int32_t* offsets,
                          int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                          const void* w_gate, const void* w_up, const void* w_down,
                          moe_dtype w_dtype,
                          const float* s_gate, const float* s_up, const float* s_down,
                          void* h, void* y_perm, void* ws, size_t ws_bytes,
                          moe_stream_t stream);

/* ------------------------------------------------------------------------
 * The two halves of moe_expert_ffn, callable on their own (moe_expert_ffn is
 * exactly moe_expert_gate_up followed by moe_expert_down on one stream).
 * Page: FusedSwiGLUExpert in "Expert implementation: SwiGLU at scale" (one
 * product over the shared input for gate and up, then w_down).
 *
 * moe_expert_gate_up: h[r,:] = silu(x[t] W_gate[e]^T) * (x[t] W_up[e]^T),
 *   t = perm[r] / k, for r in [offsets[e], offsets[e+1]); writes only h.
 *   s_gate / s_up non-NULL exactly when w_dtype is MOE_I8 or MOE_I4.
 * moe_expert_down: y_perm[r,:] = h[r,:] W_down[e]^T for the same rows.
 *   s_down non-NULL exactly when w_dtype is MOE_I8 or MOE_I4; ws as for
 *   moe_expert_ffn.
 * Arguments, layouts and rounding are those of moe_expert_ffn.
 * ------------------------------------------------------------------------ */
moe_status moe_expert_gate_up(const void* x, moe_dtype act_dtype,
                              const int32_t* perm, const int32_t* offsets,
                              int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                              const void* w_gate, const void* w_up, moe_dtype w_dtype,
                              const float* s_gate, const float* s_up, void* h,
                              moe_stream_t stream);
moe_status moe_expert_down(const void* h, moe_dtype act_dtype, const int32_t* offsets,
                           int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                           const void* w_down, moe_dtype w_dtype, const float* s_down,
                           void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Weighted combine back to token order (gather form, no atomics).
 * Page: GrokMoELayer.forward (dispatch and combine) and the expert-parallel
 * pseudocode (each expert output scaled by its routing weight).
 *
 *   out[t,:] = sum_{j=0..k-1, slot_row[t*k+j] >= 0} topk_w[t,j] * y_perm[slot_row[t*k+j],:]
 * summed in float32 in slot order j = 0, 1, ... and rounded once to act_dtype;
 * a token whose slots were all dropped gets a zero row.
 *
 * y_perm [T*k,H] (act_dtype), slot_row [T*k] int32, topk_w [T,k] float32,
 * out [T,H] (act_dtype, out).
 * ------------------------------------------------------------------------ */
moe_status moe_combine(const void* y_perm, const int32_t* slot_row, const float* topk_w,
                       int64_t T, int32_t H, int32_t k, moe_dtype act_dtype, void* out,
                       moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Routing statistics. Page: section "Routing: top-2 without auxiliary loss"
 * (the post-training expert-utilisation analysis, normalised so that a
 * balanced router scores 1.0 per expert as the page's comment intends, and
 * the remark that a clear top-2 usually stands apart from the 3rd expert
 * while the 3rd and 4th still carry noticeable probability).
 *
 * logits [T,E] float32 (in; e.g. moe_router_topk's logits output),
 * counts [E] int32 (in; moe_dispatch's counts: picks per expert before any
 * capacity drop). Outputs, each may be NULL (then not computed):
 *   utilization [E] float32: counts[e] * E / (T*k), 0 when T == 0;
 *   margin [T] float32: l_(k) - l_(k+1), the last selected logit minus the
 *     best unselected one (descending order; +inf when k == E);
 *   unselected_mass [T] float32: the probability a softmax over all E
 *     logits gives to the experts outside the top k (lower index first
 *     among equal logits; the value does not depend on that order).
 * logits may be NULL when margin and unselected_mass are; counts when
 * utilization is. Float32 arithmetic, deterministic.
 * ------------------------------------------------------------------------ */
moe_status moe_routing_stats(const float* logits, const int32_t* counts, int64_t T, int32_t E,
                             int32_t k, float* utilization, float* margin,
                             float* unselected_mass, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Expert parallelism: the layouts on either side of the all-to-all (the
 * exchange itself is the caller's, e.g. RCCL). Page: section "Expert
 * parallelism vs. tensor parallelism" (EP forward: route locally, send each
 * token to its experts' ranks, run the local experts, gather the outputs
 * back). Experts sit in contiguous blocks of E/R on R ranks (E % R == 0,
 * 1 <= R <= 64), so rows in dispatch order are grouped by destination rank.
 *
 * moe_ep_pack: send_buf[j,:] = x[perm[j] / k, :] for j < offsets[E] (the kept
 *   rows, dispatch order); send_counts[r] = rows for rank r. x [T,H] and
 *   send_buf [T*k,H] in act_dtype (16-byte aligned); perm, offsets from
 *   moe_dispatch; send_counts [R] int32.
 * moe_ep_recv_layout: recv_counts [R][E_local] int32 (rows received from
 *   source p for local expert e; the receive buffer holds source 0's rows,
 *   then source 1's, each grouped by local expert). Writes local_offsets
 *   [E_local+1] of the rows regrouped by local expert, then source, and
 *   row_index [max_rows]: the receive-buffer row of each regrouped row. The
 *   local experts then run as moe_expert_ffn(x = receive buffer, perm =
 *   row_index, offsets = local_offsets, k = 1, T = receive rows). Rows whose
 *   regrouped position would reach max_rows are not written and the offsets
 *   are capped at max_rows.
 * moe_ep_unpack: back_buf[row_index[j],:] = y_rows[j,:] for
 *   j < local_offsets[E_local]: expert outputs in receive order for the
 *   return exchange (y_rows [max_rows,H], back_buf with as many rows as the
 *   receive buffer, act_dtype, 16-byte aligned). After the exchange each
 *   source holds its rows in its own dispatch order: moe_combine's y_perm.
 * ------------------------------------------------------------------------ */
moe_status moe_ep_pack(const void* x, moe_dtype act_dtype, const int32_t* perm,
                       const int32_t* offsets, int64_t T, int32_t H, int32_t E, int32_t k,
                       int32_t R, void* send_buf, int32_t* send_counts, moe_stream_t stream);
moe_status moe_ep_recv_layout(const int32_t* recv_counts, int32_t R, int32_t E_local,
                              int64_t max_rows, int32_t* local_offsets, int32_t* row_index,
                              moe_stream_t stream);
moe_status moe_ep_unpack(const void* y_rows, moe_dtype act_dtype, const int32_t* row_index,
                         const int32_t* local_offsets, int32_t E_local, int32_t H,
                         int64_t max_rows, void* back_buf, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * The whole layer: router_topk -> dispatch -> expert_ffn -> combine on one
 * stream, with no host synchronisation. Page: GrokMoELayer.forward.
 *
 * out [T,H] (act_dtype, out). Optional outputs (each may be NULL):
 *   topk_idx [T,k] int32, topk_w [T,k] float32, counts [E] int32,
 *   offsets [E+1] int32, dropped [T*k] uint8.
 * capacity_factor <= 0 or infinite: no capacity limit (inference).
 * ws: device scratch of at least moe_layer_workspace_bytes(...) bytes; it
 * holds the routing arrays, h and y_perm between the steps, and the expert
 * FFN's scratch (moe_expert_ffn_workspace_bytes). Calls that overlap in time
 * need workspaces of their own.
 * ------------------------------------------------------------------------ */
size_t moe_layer_workspace_bytes(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                                 moe_dtype act_dtype, moe_dtype w_dtype);
moe_status moe_layer_forward(const void* x, moe_dtype act_dtype, const float* w_router,
                             const void* w_gate, const void* w_up, const void* w_down,
                             moe_dtype w_dtype,
                             const float* s_gate, const float* s_up, const float* s_down,
                             int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                             float capacity_factor, void* out,
                             int32_t* topk_idx, float* topk_w, int32_t* counts,
                             int32_t* offsets, uint8_t* dropped,
                             void* ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * The layer forward without any allocation, for callers that cannot call
 * hipMalloc or take a caller-owned workspace: code under HIP graph capture,
 * tight serving (decode) loops, harnesses that forbid allocation.
 *
 * Same arguments, checks, kernels and results as moe_layer_forward (bitwise),
 * minus ws / ws_bytes: the workspace is a fixed device array of the library,
 * MOE_NOALLOC_SCRATCH_BYTES (32 MiB), one per GPU, present from the moment
 * the library's device code is loaded on that GPU until the process ends.
 * Calls whose moe_layer_workspace_bytes(...) exceeds that size return
 * MOE_ERR_UNSUPPORTED and enqueue nothing (at the Grok-1 shape, H = 6144 and
 * F = 32768, the decode sizes T <= 16 fit: about 8.4 MiB at T = 16; larger T
 * take the tiled path, whose workspace is hundreds of MiB).
 *
 * The first call on a device looks up the array's address on that device
 * (hipGetSymbolAddress, no stream operation); later calls only read it. The
 * call allocates and frees nothing, and no part of the array needs to start
 * at zero (every call writes what it later reads).
 * Every call on one GPU shares that GPU's array and leaves the last call's
 * contents in it: calls that overlap in time on one GPU (on different
 * streams, or from different threads) race and give undefined results; use
 * moe_layer_forward with workspaces of their own for that.
 * ------------------------------------------------------------------------ */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
moe_status moe_layer_forward_noalloc(const void* x, moe_dtype act_dtype, const float* w_router,
                                     const void* w_gate, const void* w_up, const void* w_down,
                                     moe_dtype w_dtype,
                                     const float* s_gate, const float* s_up, const float* s_down,
                                     int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                                     float capacity_factor, void* out,
                                     int32_t* topk_idx, float* topk_w, int32_t* counts,
                                     int32_t* offsets, uint8_t* dropped, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Training: a forward that keeps what the backward needs, and the backward.
 * The page gives the forward (GrokMoELayer.forward) and applies the capacity
 * drop in training (grok_router_forward and the paragraph after it); the
 * backward is the exact gradient of that forward by the chain rule:
 *   - top-k selection and the capacity drop are piecewise constant: no
 *     gradient flows through them; a dropped slot adds nothing to out and
 *     gets no gradient;
 *   - for a kept slot (t,j) in dispatch row r of expert e, with
 *     g = x_t Wg_e^T, u = x_t Wu_e^T, h = silu(g) u, y = h Wd_e^T:
 *       dw[t,j] = dout_t . y,  dy = w[t,j] dout_t,  dh = dy Wd_e,
 *       dg = dh u silu'(g),  du = dh silu(g),
 *       dW_down[e] += dy^T h,  dW_gate[e] += dg^T x_t,  dW_up[e] += du^T x_t,
 *       dx_t += dg Wg_e + du Wu_e;
 *   - softmax over the selected logits:
 *       dlogit[t, idx[t,j]] = w[t,j] (dw[t,j] - sum_j' w[t,j'] dw[t,j']);
 *     then dx_t += dlogit_t W_router and dW_router = dlogit^T x.
 *
 * Supported: act_dtype = w_dtype = MOE_BF16 (else MOE_ERR_UNSUPPORTED),
 * T*k < 2^31 - 64, and the shape limits above. The expert GEMMs always run on
 * the matrix-core tiles (no decode kernels), so out may differ from
 * moe_layer_forward's in the last bf16 bit when T <= 16.
 *
 * moe_layer_forward_train: the layer forward (router, dispatch with the
 *   capacity drop, experts, combine) writing out [T,H] bf16 and the reserve:
 *   a caller-owned device buffer of moe_layer_train_reserve_bytes(...)
 *   bytes, 16-byte aligned. Its contents, each array starting on a 256-byte
 *   boundary in this order: topk_idx [T,k] int32, topk_w [T,k] float32,
 *   counts [E] int32, offsets [E+1] int32, perm [T*k] int32, slot_row [T*k]
 *   int32, dropped [T*k] uint8 (all as moe_dispatch / moe_router_topk
 *   define them), dispatch scratch (moe_dispatch_workspace_bytes), 192 MiB of
 *   expert-FFN scratch, then the
 *   bf16 pre-activations g [T*k,F] and u [T*k,F] (each rounded once from the
 *   float32 accumulator), h [T*k+64,F] and y_perm [T*k,H] (as
 *   moe_expert_ffn defines them; h has 64 rows of slack that the backward
 *   reads and masks out). Rows at or past offsets[E] are unwritten.
 * moe_layer_backward: given dout [T,H] bf16 (the gradient of out) and the
 *   reserve of the forward on the same x and weights, writes
 *   dx [T,H] bf16, dw_router [E,H] float32, dw_gate [E,F,H], dw_up [E,F,H]
 *   and dw_down [E,H,F] bf16 (every element written; zeros for an expert
 *   that received no rows). Float32 accumulation throughout; bf16 rounding
 *   of the intermediates dy, dh, [dg | du] and the per-row dx, and once of
 *   each output. ws: device scratch of moe_layer_backward_workspace_bytes
 *   (...) bytes, 16-byte aligned (it holds the row gradients dy, dh,
 *   [dg | du] and the per-row dx, and the x rows in dispatch order: about
 *   T*k*(3H + 3F)*2 bytes, plus 192 MiB of float32 partial tiles for the
 *   data-gradient products; the weights are used as stored, no transposed
 *   copies). The reserve is only read.
 * moe_layer_backward is exactly moe_layer_backward_data followed by
 *   moe_layer_backward_weights on one stream with the same reserve and ws:
 *   the data step writes dx and dw_router and leaves in ws what the weight
 *   step reads (so a schedule may run the weight step later, as long as ws
 *   and the reserve are left untouched in between); the weight step writes
 *   dw_gate, dw_up and dw_down and reads only ws and the reserve (h and the
 *   dispatch offsets), neither x nor the weights.
 * ------------------------------------------------------------------------ */
size_t moe_layer_train_reserve_bytes(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k);
size_t moe_layer_backward_workspace_bytes(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k);
moe_status moe_layer_forward_train(const void* x, moe_dtype act_dtype, const float* w_router,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   moe_dtype w_dtype, int64_t T, int32_t H, int32_t F, int32_t E,
                                   int32_t k, float capacity_factor, void* out, void* reserve,
                                   size_t reserve_bytes, moe_stream_t stream);
moe_status moe_layer_backward(const void* x, moe_dtype act_dtype, const float* w_router,
                              const void* w_gate, const void* w_up, const void* w_down,
                              moe_dtype w_dtype, int64_t T, int32_t H, int32_t F, int32_t E,
                              int32_t k, const void* dout, const void* reserve,
                              size_t reserve_bytes, void* dx, float* dw_router, void* dw_gate,
                              void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                              moe_stream_t stream);
moe_status moe_layer_backward_data(const void* x, moe_dtype act_dtype, const float* w_router,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   moe_dtype w_dtype, int64_t T, int32_t H, int32_t F, int32_t E,
                                   int32_t k, const void* dout, const void* reserve,
                                   size_t reserve_bytes, void* dx, float* dw_router, void* ws,
                                   size_t ws_bytes, moe_stream_t stream);
moe_status moe_layer_backward_weights(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                                      const void* reserve, size_t reserve_bytes, void* dw_gate,
                                      void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                                      moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
