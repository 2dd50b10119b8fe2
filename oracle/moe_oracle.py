"""Oracle for the top-2 MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow CPU reference of what the layer computes. Only the test suite,
the smoke check (__graft_entry__.smoke) and the benchmark's CPU-baseline leg
may import it; the product path (the HIP library and its Python binding)
never does.

Every function follows the n4n.ai page "How does Grok-1 use a
mixture-of-experts design?" (cited below as "the page"), written from the
page's description, not from its code listings. Precision:
  * the router product and the top-k decision are taken in float32, the
    precision the GPU kernel decides in; the same product is also formed in
    float64 to measure how close each decision was (tie flags);
  * everything else (softmax weights, expert FFN, combine) is float64 on the
    exact values the GPU consumes (bf16 widened exactly, int8 as q * s).
Library primitives used as steps: numpy matmul, argsort, exp.

Pins: tests/test_oracle_*.py check each function against brute force,
closed forms and the page's printed sizes (no function here is unpinned).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------
# storage widening (the oracle's own; exact)
# --------------------------------------------------------------------------


def widen_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 is the top half of a float32)."""
    b = np.asarray(b)
    if b.dtype != np.uint16:
        raise TypeError("bf16 values are passed as uint16 bit patterns")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


INT4_K_PER_SCALE = 128


def widen_int4(packed: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Packed int4 rows [..., K/2] (byte j: k = 2j in the low nibble, k = 2j+1
    in the high nibble; each nibble an unsigned code u, value u - 8) with one
    scale per 128 consecutive k ([..., K/128]) -> float64 [..., K]."""
    p = np.asarray(packed, np.uint8)
    codes = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.float64)
    codes[..., 0::2] = (p & 0x0F).astype(np.float64)
    codes[..., 1::2] = (p >> 4).astype(np.float64)
    s = np.repeat(np.asarray(scale, np.float32).astype(np.float64), INT4_K_PER_SCALE, axis=-1)
    if s.shape != codes.shape:
        raise ValueError("int4 scales must hold one value per row and 128 k")
    return (codes - 8.0) * s


def widen(a: np.ndarray, kind: str, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Stored matrix -> float64. kind: 'f32' | 'bf16' | 'i8' (rows scaled by
    scale[row]) | 'i4' (packed nibbles, scale per row and 128 k)."""
    if kind == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    if kind == "bf16":
        return widen_bf16_bits(a)
    if kind == "i8":
        if scale is None:
            raise ValueError("int8 weights need their per-row scales")
        # q * s is exact in float64 (8-bit times 24-bit significands)
        return np.asarray(a, np.int8).astype(np.float64) * \
            np.asarray(scale, np.float32).astype(np.float64)[:, None]
    if kind == "i4":
        if scale is None:
            raise ValueError("int4 weights need their group scales")
        return widen_int4(a, scale)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# router (the page, section "Routing: top-2 without auxiliary loss",
# grok_router_forward; and "The high-level architecture", GrokMoELayer.forward)
# --------------------------------------------------------------------------


def router_logits(x64: np.ndarray, wr: np.ndarray):
    """Bias-free router linear: logits[t,e] = sum_h x[t,h] * Wr[e,h].

    The page's router is nn.Linear(hidden, 8, bias=False) applied to the
    flattened tokens. Returns (l32, l64): the product in float32 (used for the
    decision) and in float64 (used for the softmax weights and tie gaps)."""
    wr32 = np.asarray(wr, np.float32)
    l32 = (x64.astype(np.float32) @ wr32.T).astype(np.float32)
    l64 = x64 @ wr32.astype(np.float64).T
    return l32, l64


@dataclass
class Routing:
    idx: np.ndarray      # [T,k] int32, slot 0 = larger logit
    w: np.ndarray        # [T,k] float64 softmax over the k selected logits
    tie: np.ndarray      # [T] bool: a decision gap below the tie tolerance
    l32: np.ndarray
    l64: np.ndarray


def top_k_softmax(l32: np.ndarray, l64: np.ndarray, k: int,
                  tie_tol: float = 1e-4) -> Routing:
    """Top-k experts per token and a softmax over only the selected logits.

    The page takes torch.topk over the logits (k = 2, sorted, largest first)
    and then a softmax over the k selected values. Equal logits: the lower
    expert index ranks first. A token is flagged as a tie when any of the
    decisive float64 gaps (between ranks j and j+1 for j < k, i.e. the slot
    order and the k / k+1 boundary) is below tie_tol * max(1, max|logit|)."""
    T, E = l32.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # stable sort of the negated values: equal logits keep ascending index
    order = np.argsort(-l32, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    return Routing(idx, _selected_softmax(l64, idx), _tie_flags(l64, order, k, tie_tol), l32, l64)


def _selected_softmax(l64: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits of each token, exp(l_j - l_slot0) /
    sum_j' exp(l_j' - l_slot0) (the constant subtracted does not change it)."""
    sel = np.take_along_axis(l64, np.asarray(idx, np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def _tie_flags(l64: np.ndarray, order: np.ndarray, k: int, tie_tol: float) -> np.ndarray:
    """A decisive float64 gap (ranks j, j+1 for j < k) below tie_tol * max(1, max|l|)."""
    T, E = l64.shape
    ranked64 = np.take_along_axis(l64, order, axis=1)
    last = min(k, E - 1)
    gaps = ranked64[:, :last] - ranked64[:, 1:last + 1]
    scale = np.maximum(1.0, np.abs(l64).max(axis=1)) if E > 0 else 1.0
    return (gaps < tie_tol * scale[:, None]).any(axis=1) if last > 0 else np.zeros(T, bool)


def routing_with_indices(l32: np.ndarray, l64: np.ndarray, idx: np.ndarray,
                         tie_tol: float = 1e-4) -> Routing:
    """Routing whose expert choice is given (idx [T,k], distinct per token)
    instead of taken by the top-k rule; the weights are the same softmax over
    the given selection, the tie flags those of the top-k rule.

    Where the top-k rule is decided by a gap within the tie tolerance, more
    than one choice is correct; this evaluates the layer for another such
    choice (made by an implementation that ordered the near-equal logits
    differently)."""
    idx = np.asarray(idx, np.int32)
    T, E = l32.shape
    k = idx.shape[1]
    if idx.shape[0] != T or not 1 <= k <= E:
        raise ValueError("idx must be [T,k] with 1 <= k <= E")
    if T and (idx.min() < 0 or idx.max() >= E):
        raise ValueError("expert index out of range")
    if k > 1 and T and np.any(np.diff(np.sort(idx, axis=1), axis=1) == 0):
        raise ValueError("a token selects one expert twice")
    order = np.argsort(-l32, axis=1, kind="stable")
    return Routing(idx, _selected_softmax(l64, idx), _tie_flags(l64, order, k, tie_tol), l32, l64)


# --------------------------------------------------------------------------
# dispatch with capacity (the page, grok_router_forward's one-hot dispatch
# mask and the capacity-aware dropping it applies when the factor is finite;
# capacity sizing in the paragraph after it: factor x mean load per expert)
# --------------------------------------------------------------------------


def capacity(T: int, k: int, E: int, capacity_factor) -> Optional[int]:
    """Per-expert capacity ceil(cf * (T*k) / E), evaluated in double precision
    in that order; None (no limit) when the factor is None, <= 0 or infinite.

    The page sizes capacity as the factor times the per-expert share of the
    routed work; the mean load per expert is T*k/E (section "Tradeoffs",
    expert batch size analysis)."""
    if capacity_factor is None:
        return None
    cf = float(np.float32(capacity_factor))
    if not (cf > 0) or math.isinf(cf):
        return None
    return int(math.ceil(cf * float(T * k) / float(E)))


@dataclass
class Dispatch:
    counts: np.ndarray    # [E] int32, all requests per expert (before the drop)
    offsets: np.ndarray   # [E+1] int32, exclusive scan of kept rows per expert
    perm: np.ndarray      # [T*k] int32, row -> assignment t*k+j; tail -1
    slot_row: np.ndarray  # [T*k] int32, assignment -> row, -1 if dropped
    dropped: np.ndarray   # [T*k] uint8
    cap: Optional[int]


def dispatch(idx: np.ndarray, E: int, capacity_factor=None) -> Dispatch:
    """Group assignments (t, j) by expert in token order and drop over capacity.

    Walks tokens in index order keeping one running counter per expert: an
    assignment's rank in its expert is the number of earlier tokens that chose
    that expert; it is kept iff rank < capacity. Kept rows of expert e occupy
    rows offsets[e] .. offsets[e+1]-1 in rank order."""
    T, k = idx.shape
    cap = capacity(T, k, E, capacity_factor)
    cnt = [0] * E
    rank = np.empty((T, k), np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            rank[t, j] = cnt[e]
            cnt[e] += 1
    counts = np.asarray(cnt, np.int32)
    kept = counts if cap is None else np.minimum(counts, cap)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(kept)
    perm = np.full(T * k, -1, np.int32)
    slot_row = np.full(T * k, -1, np.int32)
    dropped = np.zeros(T * k, np.uint8)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            a = t * k + j
            if cap is None or rank[t, j] < cap:
                r = int(offsets[e] + rank[t, j])
                perm[r] = a
                slot_row[a] = r
            else:
                dropped[a] = 1
    return Dispatch(counts, offsets, perm, slot_row, dropped, cap)


# --------------------------------------------------------------------------
# expert FFN (the page, section "Expert implementation: SwiGLU at scale",
# SwiGLUExpert: w_down(silu(w_gate x) * w_up x), all bias-free)
# --------------------------------------------------------------------------


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_hidden(x64: np.ndarray, wg64: np.ndarray, wu64: np.ndarray) -> np.ndarray:
    """The expert's hidden activation on rows x [m,H]: silu(x Wg^T) * (x Wu^T) -> [m,F]."""
    return silu(x64 @ wg64.T) * (x64 @ wu64.T)


def swiglu_expert(x64: np.ndarray, wg64: np.ndarray, wu64: np.ndarray,
                  wd64: np.ndarray) -> np.ndarray:
    """One expert on rows x [m,H]: (silu(x Wg^T) * (x Wu^T)) Wd^T -> [m,H]."""
    return expert_hidden(x64, wg64, wu64) @ wd64.T


def combine(y_rows: np.ndarray, slot_row: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Weighted combine back to token order: out[t] = sum over slots j with
    slot_row[t*k+j] >= 0 of w[t,j] * y_rows[slot_row[t*k+j]], slot 0 first;
    zero rows for tokens whose slots were all dropped (GrokMoELayer.forward;
    the EP pseudocode scales each expert output by the token's weight)."""
    T, k = w.shape
    out = np.zeros((T, y_rows.shape[1]), np.float64)
    for t in range(T):
        for j in range(k):
            r = int(slot_row[t * k + j])
            if r >= 0:
                out[t] += float(w[t, j]) * y_rows[r].astype(np.float64)
    return out


# --------------------------------------------------------------------------
# the layer (the page, GrokMoELayer.forward: flatten, router, top-2, softmax
# over the selected logits, per-expert compute and weighted combine; the EP
# pseudocode in "Expert parallelism vs. tensor parallelism" multiplies each
# expert's output by the token's weight for that expert and skips experts
# that received no token)
# --------------------------------------------------------------------------


@dataclass
class LayerResult:
    routing: Routing
    disp: Dispatch
    tokens: np.ndarray    # token ids whose outputs were evaluated
    out: np.ndarray       # [len(tokens), H] float64


def layer_forward(x: np.ndarray, act: str, wr: np.ndarray,
                  wg: Sequence, wu: Sequence, wd: Sequence, wdt: str,
                  k: int = 2, capacity_factor=None,
                  sg=None, su=None, sd=None,
                  tokens: Optional[np.ndarray] = None,
                  tie_tol: float = 1e-4, idx: Optional[np.ndarray] = None) -> LayerResult:
    """Whole-layer forward. Routing and dispatch run over all T tokens (the
    capacity decision depends on every earlier token); the expert FFN and the
    combine run only for `tokens` (all tokens when None).

    out[t] = sum over kept slots j of w[t,j] * expert_{idx[t,j]}(x[t]),
    slot 0 first; a token whose slots were all dropped gets a zero row.
    idx: the experts chosen per token, when given (routing_with_indices);
    otherwise the top-k rule chooses."""
    x64 = widen(x, act)
    T, H = x64.shape
    E = np.asarray(wr).shape[0]
    l32, l64 = router_logits(x64, wr)
    routing = top_k_softmax(l32, l64, k, tie_tol) if idx is None else \
        routing_with_indices(l32, l64, idx, tie_tol)
    disp = dispatch(routing.idx, E, capacity_factor)

    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    # expert output of every kept (sample position, slot) pair
    y_of = {}
    for e in range(E):
        pairs = [(p, j) for p, t in enumerate(tokens) for j in range(k)
                 if routing.idx[t, j] == e and disp.slot_row[t * k + j] >= 0]
        if not pairs:
            continue          # an expert that received no tokens is skipped
        s_g = None if sg is None else sg[e]
        s_u = None if su is None else su[e]
        s_d = None if sd is None else sd[e]
        y = swiglu_expert(x64[[int(tokens[p]) for p, _ in pairs]],
                          widen(wg[e], wdt, s_g), widen(wu[e], wdt, s_u),
                          widen(wd[e], wdt, s_d))
        for i, pj in enumerate(pairs):
            y_of[pj] = y[i]
    # weighted combine back to token order, slot 0 first
    out = np.zeros((len(tokens), H), np.float64)
    for p, t in enumerate(tokens):
        for j in range(k):
            if (p, j) in y_of:
                out[p] += routing.w[t, j] * y_of[(p, j)]
    return LayerResult(routing, disp, tokens, out)


# --------------------------------------------------------------------------
# the layer's backward (training). The page gives the forward only and marks
# the capacity drop as a training-time step; the backward here is the chain
# rule applied to that forward, taken exactly: the top-k choice and the
# capacity drop are piecewise constant in the inputs, so no gradient flows
# through the selection; a dropped slot contributes nothing to the output
# and so receives no gradient; the routing weights are a softmax over the k
# selected logits, whose Jacobian couples the selected slots of a token.
# --------------------------------------------------------------------------


def silu_grad(g: np.ndarray) -> np.ndarray:
    """d silu / dg = s + g s (1 - s), s = 1 / (1 + exp(-g))."""
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    return s + g * s * (1.0 - s)


@dataclass
class LayerGrads:
    routing: Routing
    disp: Dispatch
    out: np.ndarray      # [T,H] forward output
    dx: np.ndarray       # [T,H]
    dwr: np.ndarray      # [E,H]
    dwg: np.ndarray      # [E,F,H]
    dwu: np.ndarray      # [E,F,H]
    dwd: np.ndarray      # [E,H,F]
    dw: np.ndarray       # [T,k] gradient of the routing weights (0 for dropped slots)
    dlogits: np.ndarray  # [T,E] gradient of the router logits


def layer_backward(x: np.ndarray, act: str, wr: np.ndarray,
                   wg: Sequence, wu: Sequence, wd: Sequence, wdt: str,
                   dout: np.ndarray, k: int = 2, capacity_factor=None,
                   tie_tol: float = 1e-4, idx: Optional[np.ndarray] = None) -> LayerGrads:
    """Gradients of L = sum(dout * out) for the layer of layer_forward, in
    float64 on the stored values (routing decided as in layer_forward).

    For a kept slot (t, j) routed to expert e, with row x_t:
      g = x_t Wg_e^T, u = x_t Wu_e^T, h = silu(g) * u, y = h Wd_e^T
      dw[t,j]  = dout_t . y                     (out_t = sum_j w[t,j] y_(t,j))
      dy       = w[t,j] * dout_t
      dh       = dy Wd_e
      dg       = dh * u * silu'(g),  du = dh * silu(g)
      dWd_e   += dy^T h,  dWg_e += dg^T x_t,  dWu_e += du^T x_t
      dx_t    += dg Wg_e + du Wu_e
    Softmax over the selected logits, w_j = exp(l_j) / sum_j' exp(l_j'):
      dl[t, idx[t,j]] = w_j (dw_j - sum_j' w_j' dw_j'), zero for unselected
    Router, logits = x Wr^T:  dx_t += dl_t Wr,  dWr = dl^T x.
    idx: the experts chosen per token, when given (as in layer_forward)."""
    x64 = widen(x, act)
    T, H = x64.shape
    wr64 = np.asarray(wr, np.float32).astype(np.float64)
    E = wr64.shape[0]
    d64 = np.asarray(dout, np.float64)
    l32, l64 = router_logits(x64, wr)
    routing = top_k_softmax(l32, l64, k, tie_tol) if idx is None else \
        routing_with_indices(l32, l64, idx, tie_tol)
    disp = dispatch(routing.idx, E, capacity_factor)

    F = widen(wg[0], wdt).shape[0]
    out = np.zeros((T, H))
    dx = np.zeros((T, H))
    dwg = np.zeros((E, F, H))
    dwu = np.zeros((E, F, H))
    dwd = np.zeros((E, H, F))
    dw = np.zeros((T, k))
    for e in range(E):
        # the expert's kept slots in dispatch order
        rows = range(int(disp.offsets[e]), int(disp.offsets[e + 1]))
        slots = [int(disp.perm[r]) for r in rows]
        if not slots:
            continue
        ts = np.array([a // k for a in slots])
        js = np.array([a % k for a in slots])
        Wg, Wu, Wd = widen(wg[e], wdt), widen(wu[e], wdt), widen(wd[e], wdt)
        X = x64[ts]
        g = X @ Wg.T
        u = X @ Wu.T
        h = silu(g) * u
        y = h @ Wd.T
        wts = routing.w[ts, js]
        out[ts] += wts[:, None] * y          # distinct slots: (t, j) pairs are unique
        dw[ts, js] = np.sum(d64[ts] * y, axis=1)
        dy = wts[:, None] * d64[ts]
        dh = dy @ Wd
        dg = dh * u * silu_grad(g)
        du = dh * silu(g)
        dwd[e] = dy.T @ h
        dwg[e] = dg.T @ X
        dwu[e] = du.T @ X
        np.add.at(dx, ts, dg @ Wg + du @ Wu)
    # softmax over the selected logits
    s = np.sum(routing.w * dw, axis=1, keepdims=True)
    dsel = routing.w * (dw - s)
    dl = np.zeros((T, E))
    np.put_along_axis(dl, routing.idx.astype(np.int64), dsel, axis=1)
    dx += dl @ wr64
    dwr = dl.T @ x64
    return LayerGrads(routing, disp, out, dx, dwr, dwg, dwu, dwd, dw, dl)


@dataclass
class SampledGrads:
    routing: Routing
    disp: Dispatch
    tokens: np.ndarray   # sampled tokens
    dx: np.ndarray       # [len(tokens), H]
    entries: dict        # name -> (indices [n,3] (e, row, col), values [n])
    dwr: Optional[np.ndarray] = None   # [E,H] router weight gradient (router_grad=True)


def layer_backward_sampled(x: np.ndarray, act: str, wr: np.ndarray,
                           wg: Sequence, wu: Sequence, wd: Sequence, wdt: str,
                           dout: np.ndarray, k: int, capacity_factor, tokens: np.ndarray,
                           entries: dict, tie_tol: float = 1e-4,
                           idx: Optional[np.ndarray] = None, router_grad: bool = False,
                           progress=None) -> SampledGrads:
    """Selected outputs of layer_backward at sizes where the whole backward
    is too slow on the CPU: dx for `tokens`, and the weight-gradient entries
    entries[name] = [(e, i, j), ...] for name in dwg / dwu ([e][f][h]) and
    dwd ([e][h][f]). Same formulas, evaluated per entry in float64:
      dWd[e][h][f] = sum over e's rows r of dy_r[h] h_r[f]
      dWg[e][f][h] = sum_r dg_r[f] x_r[h],  dWu[e][f][h] = sum_r du_r[f] x_r[h]
    with h_r[f], dg_r[f], du_r[f] from column f of W_gate / W_up / W_down,
    and dx_t as in layer_backward (the token's own slots and its logits).
    Expert weights are read one expert at a time (wg[e] etc. may be lazy).

    router_grad=True also gives the whole router weight gradient dWr = dl^T x,
    which needs dw[t,j] = dout_t . y_(t,j) for every kept slot: each expert's
    output rows are then evaluated for all of its rows (the full forward).
    idx: the experts chosen per token, when given (as in layer_forward).
    progress: optional callable taking a message, called once per expert."""
    x64 = widen(x, act)
    T, H = x64.shape
    wr64 = np.asarray(wr, np.float32).astype(np.float64)
    E = wr64.shape[0]
    l32, l64 = router_logits(x64, wr)
    routing = top_k_softmax(l32, l64, k, tie_tol) if idx is None else \
        routing_with_indices(l32, l64, idx, tie_tol)
    disp = dispatch(routing.idx, E, capacity_factor)
    tokens = np.asarray(tokens, np.int64)

    def d64(t):
        return np.asarray(dout[t], np.float64)

    dx = np.zeros((len(tokens), H))
    dw_tok = np.zeros((len(tokens), k))
    dw_all = np.zeros((T, k)) if router_grad else None
    vals = {n: np.zeros(len(v)) for n, v in entries.items()}
    for e in range(E):
        rows = range(int(disp.offsets[e]), int(disp.offsets[e + 1]))
        slots = np.array([int(disp.perm[r]) for r in rows], np.int64)
        mine = {n: [i for i, (ee, _, _) in enumerate(v) if ee == e] for n, v in entries.items()}
        tok_slots = [(p, j) for p, t in enumerate(tokens) for j in range(k)
                     if routing.idx[t, j] == e and disp.slot_row[t * k + j] >= 0]
        if len(slots) == 0 or (not any(mine.values()) and not tok_slots and not router_grad):
            continue
        if progress is not None:
            progress(f"oracle backward: expert {e}, {len(slots)} rows")
        ts, js = slots // k, slots % k
        X = x64[ts]
        wts = routing.w[ts, js]
        D = np.stack([d64(t) for t in ts]) if len(ts) else np.zeros((0, H))
        dy = wts[:, None] * D
        Wg, Wu, Wd = widen(wg[e], wdt), widen(wu[e], wdt), widen(wd[e], wdt)
        if router_grad:
            # dw of every kept slot of this expert: dout_t . y, y = h Wd^T
            y = (silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
            dw_all[ts, js] = np.sum(D * y, axis=1)
            del y
        # entries: per-column quantities over all of the expert's rows
        for n, ids in mine.items():
            for i in ids:
                _, a, b = entries[n][i]
                if n == "dwd":               # [e][h = a][f = b]
                    g, u = X @ Wg[b], X @ Wu[b]
                    vals[n][i] = np.sum(dy[:, a] * silu(g) * u)
                else:                        # [e][f = a][h = b]
                    g, u = X @ Wg[a], X @ Wu[a]
                    dh = dy @ Wd[:, a]
                    col = dh * u * silu_grad(g) if n == "dwg" else dh * silu(g)
                    vals[n][i] = np.sum(col * X[:, b])
        # the sampled tokens' own slots: whole rows, all of this expert's at once
        if tok_slots:
            ps = np.array([p for p, _ in tok_slots], np.int64)
            jsl = np.array([j for _, j in tok_slots], np.int64)
            tt = tokens[ps]
            g, u = x64[tt] @ Wg.T, x64[tt] @ Wu.T
            y = (silu(g) * u) @ Wd.T
            Ds = np.stack([d64(t) for t in tt])
            dw_tok[ps, jsl] = np.sum(Ds * y, axis=1)
            dh = (routing.w[tt, jsl][:, None] * Ds) @ Wd
            np.add.at(dx, ps, (dh * u * silu_grad(g)) @ Wg + (dh * silu(g)) @ Wu)
    for p, t in enumerate(tokens):
        w = routing.w[t]
        dsel = w * (dw_tok[p] - np.sum(w * dw_tok[p]))
        dx[p] += dsel @ wr64[routing.idx[t].astype(np.int64)]
    ent = {n: (np.asarray(v, np.int64).reshape(-1, 3), vals[n]) for n, v in entries.items()}
    dwr = None
    if router_grad:
        # softmax over the selected logits of every token, then dWr = dl^T x
        dsel = routing.w * (dw_all - np.sum(routing.w * dw_all, axis=1, keepdims=True))
        dl = np.zeros((T, E))
        np.put_along_axis(dl, routing.idx.astype(np.int64), dsel, axis=1)
        dwr = dl.T @ x64
    return SampledGrads(routing, disp, tokens, dx, ent, dwr)


# --------------------------------------------------------------------------
# sizes and statistics printed or used on the page
# --------------------------------------------------------------------------


def mean_rows_per_expert(T: int, k: int, E: int) -> float:
    """Rows an expert receives on average: the T*k assignments spread over E
    experts (the expert batch sizes of section "Tradeoffs: when MoE wins and
    when it doesn't", whose token count is batch * sequence length)."""
    return T * k / E


def expert_params(hidden: int, expert_dim: int) -> int:
    """Weights of one SwiGLU expert: gate and up [F,H] plus down [H,F]."""
    return 3 * hidden * expert_dim


def expert_utilization(idx: np.ndarray, E: int) -> np.ndarray:
    """Per-expert share of the top-k picks normalised so a balanced router
    scores 1.0 for every expert: counts / (T*k) * E. (The page's utilisation
    snippet divides by the number of picks and then multiplies by E/2, which
    gives 0.5 for a balanced router, not the 1.0 its comment claims; this is
    the normalisation the comment describes.)"""
    idx = np.asarray(idx)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.float64)
    return counts / idx.size * E


@dataclass
class RoutingStats:
    margin: np.ndarray           # [T] l_(k) - l_(k+1); +inf when k == E
    unselected_mass: np.ndarray  # [T] full-softmax probability outside the top k
    utilization: np.ndarray      # [E] counts / (T*k) * E


def routing_stats(l32: np.ndarray, k: int, counts: np.ndarray) -> RoutingStats:
    """Routing statistics the page discusses after training (section
    "Routing: top-2 without auxiliary loss", the utilisation analysis and the
    remark that a clear top-2 usually stands apart from the 3rd expert, while
    the 3rd and 4th still carry noticeable probability).

    Per token: the margin between the last selected logit and the best
    unselected one, l_(k) - l_(k+1) (values in descending order; the order of
    equal values does not matter here), and the probability a softmax over
    all E logits gives to the experts outside the top k. Per expert: the
    picks counted by the dispatch, normalised as in expert_utilization. All in
    float64 from the float32 logits."""
    l = np.asarray(l32, np.float32).astype(np.float64)
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ranked = -np.sort(-l, axis=1)
    margin = ranked[:, k - 1] - ranked[:, k] if k < E else np.full(T, np.inf)
    z = np.exp(l - ranked[:, :1])
    # the selected set: k largest, lower index first among equal values
    order = np.argsort(-np.asarray(l32, np.float32), axis=1, kind="stable")
    outside = np.ones_like(z, bool)
    np.put_along_axis(outside, order[:, :k], False, axis=1)
    mass = (z * outside).sum(axis=1) / z.sum(axis=1) if T else np.zeros(0)
    counts = np.asarray(counts, np.float64)
    util = counts * E / (T * k) if T else np.zeros(E)
    return RoutingStats(margin, mass, util)


# --------------------------------------------------------------------------
# expert parallelism: the data movement around the all-to-all (the page,
# section "Expert parallelism vs. tensor parallelism": EP places whole
# experts on ranks; each rank routes its own tokens, sends them to the ranks
# of their experts, runs its local experts and gathers the outputs back).
# Experts are placed in contiguous blocks: rank r holds E/R experts
# r*E/R ... (r+1)*E/R - 1. The exchange itself is not modelled here; these
# are the layouts on either side of it.
# --------------------------------------------------------------------------


def ep_pack(x: np.ndarray, perm: np.ndarray, offsets: np.ndarray, k: int, E: int, R: int):
    """Rows a rank sends: the x row of every kept assignment, in dispatch
    order (grouped by expert, hence by destination rank), and the number of
    rows for each destination rank."""
    if E % R:
        raise ValueError("E must be a multiple of R")
    n = int(offsets[E])
    rows = np.asarray(x)[np.asarray(perm[:n], np.int64) // k]
    per = E // R
    counts = np.array([offsets[(r + 1) * per] - offsets[r * per] for r in range(R)], np.int64)
    return rows, counts


def ep_recv_layout(recv_counts: np.ndarray):
    """recv_counts[p][e]: rows received from source rank p for local expert e
    (the receive buffer holds source 0's rows, then source 1's, ..., each
    source's rows grouped by local expert). Returns (offsets [E_local+1] of
    the rows regrouped by local expert, then source; row_index: for each
    regrouped row, its position in the receive buffer)."""
    c = np.asarray(recv_counts, np.int64)
    R, El = c.shape
    start = np.zeros((R, El), np.int64)
    pos = 0
    for p in range(R):
        for e in range(El):
            start[p, e] = pos
            pos += c[p, e]
    row_index, offsets = [], [0]
    for e in range(El):
        for p in range(R):
            row_index.extend(range(start[p, e], start[p, e] + c[p, e]))
        offsets.append(len(row_index))
    return np.array(offsets, np.int64), np.array(row_index, np.int64)


def ep_unpack(y_rows: np.ndarray, row_index: np.ndarray, n_recv: int) -> np.ndarray:
    """Expert outputs (regrouped order) back to receive-buffer order, ready
    for the return exchange: back[row_index[j]] = y_rows[j]."""
    y_rows = np.asarray(y_rows)
    back = np.zeros((n_recv,) + y_rows.shape[1:], y_rows.dtype)
    back[np.asarray(row_index, np.int64)] = y_rows
    return back

