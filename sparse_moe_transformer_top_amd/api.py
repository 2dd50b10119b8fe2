"""Python binding of the layer's C ABI (torch tensors in, torch tensors out).

Argument marshalling only: shapes and dtypes are read off the tensors, output
buffers are allocated with torch on the input's device, and each function
makes exactly one call into libmoe.so on torch's current stream. Every step
of the layer runs in the library's HIP kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import MOE_BF16, MOE_F32, MOE_I4, MOE_I8, check

# int4 weights travel as packed bytes (two codes per byte) in uint8 tensors
_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.int8: MOE_I8, torch.uint8: MOE_I4}
_WDT = (torch.float32, torch.bfloat16, torch.int8, torch.uint8)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions")


def _cf(capacity_factor) -> float:
    return 0.0 if capacity_factor is None else float(capacity_factor)


def moe_router_topk(x: torch.Tensor, w_router: torch.Tensor, k: int = 2,
                    return_logits: bool = False):
    """(topk_idx [T,k] int32, topk_w [T,k] float32[, logits [T,E] float32])."""
    _need(x, "x", (torch.float32, torch.bfloat16), 2)
    _need(w_router, "w_router", torch.float32, 2)
    T, H = x.shape
    E = w_router.shape[0]
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if return_logits else None
    check(_lib.load().moe_router_topk(_p(x), _DT[x.dtype], _p(w_router), T, H, E, k, _p(idx),
                                      _p(w), _p(logits), _stream(x.device)))
    return (idx, w, logits) if return_logits else (idx, w)


def moe_dispatch(topk_idx: torch.Tensor, E: int, capacity_factor: Optional[float] = None):
    """dict(counts [E], offsets [E+1], perm [T*k], slot_row [T*k] int32, dropped [T*k] uint8)."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    T, k = topk_idx.shape
    dev = topk_idx.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
               perm=torch.empty(T * k, **i32), slot_row=torch.empty(T * k, **i32),
               dropped=torch.empty(T * k, dtype=torch.uint8, device=dev))
    lib = _lib.load()
    nws = lib.moe_dispatch_workspace_bytes(T, E, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    check(lib.moe_dispatch(_p(topk_idx), T, E, k, _cf(capacity_factor), _p(out["counts"]),
                           _p(out["offsets"]), _p(out["perm"]), _p(out["slot_row"]),
                           _p(out["dropped"]), _p(ws), nws, _stream(dev)))
    return out


def moe_expert_ffn(x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor, k: int,
                   w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                   s_gate=None, s_up=None, s_down=None):
    """(h [T*k,F], y_perm [T*k,H]) in x's dtype; rows past offsets[E] are unwritten."""
    _need(x, "x", (torch.float32, torch.bfloat16), 2)
    for n, t in (("perm", perm), ("offsets", offsets)):
        _need(t, n, torch.int32, 1)
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, n, _WDT, 3)
    T, H = x.shape
    E, F, _ = w_gate.shape
    h = torch.empty((T * k, F), dtype=x.dtype, device=x.device)
    y = torch.empty((T * k, H), dtype=x.dtype, device=x.device)
    lib = _lib.load()
    nws = lib.moe_expert_ffn_workspace_bytes(T, H, F, E, k, _DT[x.dtype], _DT[w_gate.dtype])
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device)
    check(lib.moe_expert_ffn(_p(x), _DT[x.dtype], _p(perm), _p(offsets), T, H, F, E, k,
                             _p(w_gate), _p(w_up), _p(w_down), _DT[w_gate.dtype], _p(s_gate),
                             _p(s_up), _p(s_down), _p(h), _p(y), _p(ws), nws, _stream(x.device)))
    return h, y


def moe_expert_gate_up(x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor, k: int,
                       w_gate: torch.Tensor, w_up: torch.Tensor, s_gate=None, s_up=None,
                       h: Optional[torch.Tensor] = None):
    """h [T*k,F] = silu(x W_gate^T) * (x W_up^T) over the dispatched rows."""
    _need(x, "x", (torch.float32, torch.bfloat16), 2)
    T, H = x.shape
    E, F, _ = w_gate.shape
    if h is None:
        h = torch.empty((T * k, F), dtype=x.dtype, device=x.device)
    check(_lib.load().moe_expert_gate_up(_p(x), _DT[x.dtype], _p(perm), _p(offsets), T, H, F, E,
                                         k, _p(w_gate), _p(w_up), _DT[w_gate.dtype], _p(s_gate),
                                         _p(s_up), _p(h), _stream(x.device)))
    return h


def moe_expert_down(h: torch.Tensor, offsets: torch.Tensor, T: int, k: int,
                    w_down: torch.Tensor, s_down=None, y_perm: Optional[torch.Tensor] = None):
    """y_perm [T*k,H] = h W_down^T over the dispatched rows."""
    _need(h, "h", (torch.float32, torch.bfloat16), 2)
    _need(w_down, "w_down", _WDT, 3)
    E, H, F = w_down.shape
    if w_down.dtype == torch.uint8:
        F *= 2                       # packed int4: two k per byte
    if y_perm is None:
        y_perm = torch.empty((T * k, H), dtype=h.dtype, device=h.device)
    lib = _lib.load()
    nws = lib.moe_expert_ffn_workspace_bytes(T, H, F, E, k, _DT[h.dtype], _DT[w_down.dtype])
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=h.device)
    check(lib.moe_expert_down(_p(h), _DT[h.dtype], _p(offsets), T, H, F, E, k, _p(w_down),
                              _DT[w_down.dtype], _p(s_down), _p(y_perm), _p(ws), nws,
                              _stream(h.device)))
    return y_perm


def moe_combine(y_perm: torch.Tensor, slot_row: torch.Tensor, topk_w: torch.Tensor):
    """out [T,H] in y_perm's dtype."""
    _need(y_perm, "y_perm", (torch.float32, torch.bfloat16), 2)
    _need(slot_row, "slot_row", torch.int32, 1)
    _need(topk_w, "topk_w", torch.float32, 2)
    T, k = topk_w.shape
    H = y_perm.shape[1]
    out = torch.empty((T, H), dtype=y_perm.dtype, device=y_perm.device)
    check(_lib.load().moe_combine(_p(y_perm), _p(slot_row), _p(topk_w), T, H, k,
                                  _DT[y_perm.dtype], _p(out), _stream(y_perm.device)))
    return out


def moe_routing_stats(logits: torch.Tensor, counts: torch.Tensor, k: int):
    """dict(utilization [E], margin [T], unselected_mass [T]) float32 from
    logits [T,E] float32 and the dispatch counts [E] int32."""
    _need(logits, "logits", torch.float32, 2)
    _need(counts, "counts", torch.int32, 1)
    T, E = logits.shape
    f32 = dict(dtype=torch.float32, device=logits.device)
    out = dict(utilization=torch.empty(E, **f32), margin=torch.empty(T, **f32),
               unselected_mass=torch.empty(T, **f32))
    check(_lib.load().moe_routing_stats(_p(logits), _p(counts), T, E, k, _p(out["utilization"]),
                                        _p(out["margin"]), _p(out["unselected_mass"]),
                                        _stream(logits.device)))
    return out


def moe_ep_pack(x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor, k: int, R: int):
    """(send_buf [T*k,H] in x's dtype: the kept rows in dispatch order, rows past
    offsets[E] unwritten; send_counts [R] int32: rows for each rank)."""
    _need(x, "x", (torch.float32, torch.bfloat16), 2)
    T, H = x.shape
    E = offsets.numel() - 1
    send = torch.empty((T * k, H), dtype=x.dtype, device=x.device)
    counts = torch.empty(R, dtype=torch.int32, device=x.device)
    check(_lib.load().moe_ep_pack(_p(x), _DT[x.dtype], _p(perm), _p(offsets), T, H, E, k, R,
                                  _p(send), _p(counts), _stream(x.device)))
    return send, counts


def moe_ep_recv_layout(recv_counts: torch.Tensor, max_rows: int):
    """(local_offsets [E_local+1], row_index [max_rows]) int32 from
    recv_counts [R, E_local] int32."""
    _need(recv_counts, "recv_counts", torch.int32, 2)
    R, El = recv_counts.shape
    dev = recv_counts.device
    off = torch.empty(El + 1, dtype=torch.int32, device=dev)
    idx = torch.empty(max(max_rows, 1), dtype=torch.int32, device=dev)
    check(_lib.load().moe_ep_recv_layout(_p(recv_counts), R, El, max_rows, _p(off), _p(idx),
                                         _stream(dev)))
    return off, idx[:max_rows]


def moe_ep_unpack(y_rows: torch.Tensor, row_index: torch.Tensor, local_offsets: torch.Tensor,
                  n_recv: int):
    """back [n_recv, H]: back[row_index[j]] = y_rows[j] for j < local_offsets[-1]."""
    _need(y_rows, "y_rows", (torch.float32, torch.bfloat16), 2)
    max_rows, H = y_rows.shape
    back = torch.empty((n_recv, H), dtype=y_rows.dtype, device=y_rows.device)
    check(_lib.load().moe_ep_unpack(_p(y_rows), _DT[y_rows.dtype], _p(row_index),
                                    _p(local_offsets), local_offsets.numel() - 1, H, max_rows,
                                    _p(back), _stream(y_rows.device)))
    return back


def layer_workspace_bytes(T: int, H: int, F: int, E: int, k: int, act: torch.dtype,
                          wdt: torch.dtype) -> int:
    return _lib.load().moe_layer_workspace_bytes(T, H, F, E, k, _DT[act], _DT[wdt])


def moe_layer_forward(x: torch.Tensor, w_router: torch.Tensor, w_gate: torch.Tensor,
                      w_up: torch.Tensor, w_down: torch.Tensor, k: int = 2,
                      capacity_factor: Optional[float] = None, s_gate=None, s_up=None,
                      s_down=None, workspace: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, aux: bool = False):
    """The whole layer. Returns out [T,H], or (out, dict of routing outputs) with aux=True."""
    _need(x, "x", (torch.float32, torch.bfloat16), 2)
    _need(w_router, "w_router", torch.float32, 2)
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, n, _WDT, 3)
    T, H = x.shape
    E, F, _ = w_gate.shape
    dev = x.device
    nws = layer_workspace_bytes(T, H, F, E, k, x.dtype, w_gate.dtype)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    ax = None
    if aux:
        i32 = dict(dtype=torch.int32, device=dev)
        ax = dict(topk_idx=torch.empty((T, k), **i32),
                  topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
                  counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                  dropped=torch.empty(T * k, dtype=torch.uint8, device=dev))
    g = (lambda n: None if ax is None else _p(ax[n]))
    check(_lib.load().moe_layer_forward(
        _p(x), _DT[x.dtype], _p(w_router), _p(w_gate), _p(w_up), _p(w_down), _DT[w_gate.dtype],
        _p(s_gate), _p(s_up), _p(s_down), T, H, F, E, k, _cf(capacity_factor), _p(out),
        g("topk_idx"), g("topk_w"), g("counts"), g("offsets"), g("dropped"), _p(workspace),
        workspace.numel(), _stream(dev)))
    return (out, ax) if aux else out


def moe_layer_forward_noalloc(x: torch.Tensor, w_router: torch.Tensor, w_gate: torch.Tensor,
                              w_up: torch.Tensor, w_down: torch.Tensor, k: int = 2,
                              capacity_factor: Optional[float] = None, s_gate=None, s_up=None,
                              s_down=None, out: Optional[torch.Tensor] = None,
                              aux: Optional[dict] = None):
    """moe_layer_forward on the library's fixed scratch array instead of a
    workspace (no allocation by the library; shapes whose workspace exceeds
    NOALLOC_SCRATCH_BYTES are rejected). out and the aux buffers (topk_idx,
    topk_w, counts, offsets, dropped, each optional) are the caller's, so a
    call with them given allocates nothing. Returns out."""
    _need(x, "x", (torch.float32, torch.bfloat16), 2)
    _need(w_router, "w_router", torch.float32, 2)
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, n, _WDT, 3)
    T, H = x.shape
    E, F, _ = w_gate.shape
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=x.device)
    _need(out, "out", x.dtype, 2)
    ax = aux or {}
    g = (lambda n: _p(ax.get(n)))
    check(_lib.load().moe_layer_forward_noalloc(
        _p(x), _DT[x.dtype], _p(w_router), _p(w_gate), _p(w_up), _p(w_down), _DT[w_gate.dtype],
        _p(s_gate), _p(s_up), _p(s_down), T, H, F, E, k, _cf(capacity_factor), _p(out),
        g("topk_idx"), g("topk_w"), g("counts"), g("offsets"), g("dropped"), _stream(x.device)))
    return out


def train_reserve_bytes(T: int, H: int, F: int, E: int, k: int) -> int:
    return _lib.load().moe_layer_train_reserve_bytes(T, H, F, E, k)


def backward_workspace_bytes(T: int, H: int, F: int, E: int, k: int) -> int:
    return _lib.load().moe_layer_backward_workspace_bytes(T, H, F, E, k)


# expert-FFN scratch in the training reserve (include/moe.h: 192 MiB)
FFN_SCRATCH_BYTES = 192 << 20


def _align256(n: int) -> int:
    return (n + 255) // 256 * 256


def train_reserve_views(reserve: torch.Tensor, T: int, H: int, F: int, E: int, k: int):
    """Views of the arrays moe_layer_forward_train keeps in the reserve (the
    layout include/moe.h documents): routing, dispatch, g, u, h (its T*k
    rows; 64 slack rows follow), y_perm."""
    N = T * k
    disp_ws = _lib.load().moe_dispatch_workspace_bytes(T, E, k)
    parts = [("topk_idx", torch.int32, (T, k)), ("topk_w", torch.float32, (T, k)),
             ("counts", torch.int32, (E,)), ("offsets", torch.int32, (E + 1,)),
             ("perm", torch.int32, (N,)), ("slot_row", torch.int32, (N,)),
             ("dropped", torch.uint8, (N,)), ("dispatch_scratch", torch.uint8, (disp_ws,)),
             ("ffn_scratch", torch.uint8, (FFN_SCRATCH_BYTES,)),
             ("g", torch.bfloat16, (N, F)), ("u", torch.bfloat16, (N, F)),
             ("h", torch.bfloat16, (N + 64, F)), ("y_perm", torch.bfloat16, (N, H))]
    out, off = {}, 0
    for name, dt, shape in parts:
        n = 1
        for d in shape:
            n *= d
        nbytes = n * torch.empty((), dtype=dt).element_size()
        out[name] = reserve[off:off + nbytes].view(dt).view(shape)[:N] if name == "h" else \
            reserve[off:off + nbytes].view(dt).view(shape)
        off += _align256(nbytes)
    return out


def moe_layer_forward_train(x: torch.Tensor, w_router: torch.Tensor, w_gate: torch.Tensor,
                            w_up: torch.Tensor, w_down: torch.Tensor, k: int = 2,
                            capacity_factor: Optional[float] = None,
                            reserve: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None):
    """Training forward (bf16). Returns (out [T,H], reserve): the reserve
    (uint8 device buffer) holds what moe_layer_backward reads."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_router, "w_router", torch.float32, 2)
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, n, torch.bfloat16, 3)
    T, H = x.shape
    E, F, _ = w_gate.shape
    dev = x.device
    nres = train_reserve_bytes(T, H, F, E, k)
    if reserve is None or reserve.numel() < nres:
        reserve = torch.empty(max(nres, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    check(_lib.load().moe_layer_forward_train(
        _p(x), MOE_BF16, _p(w_router), _p(w_gate), _p(w_up), _p(w_down), MOE_BF16, T, H, F, E, k,
        _cf(capacity_factor), _p(out), _p(reserve), reserve.numel(), _stream(dev)))
    return out, reserve


def moe_layer_backward(x: torch.Tensor, w_router: torch.Tensor, w_gate: torch.Tensor,
                       w_up: torch.Tensor, w_down: torch.Tensor, dout: torch.Tensor,
                       reserve: torch.Tensor, k: int = 2,
                       workspace: Optional[torch.Tensor] = None, grads: Optional[dict] = None,
                       split: bool = False):
    """Backward of moe_layer_forward_train. Returns a dict with dx [T,H] bf16,
    dw_router [E,H] float32, dw_gate, dw_up [E,F,H] and dw_down [E,H,F] bf16
    (written into `grads` when given). split=True makes the same computation
    as two calls, moe_layer_backward_data then moe_layer_backward_weights."""
    _need(x, "x", torch.bfloat16, 2)
    _need(dout, "dout", torch.bfloat16, 2)
    _need(w_router, "w_router", torch.float32, 2)
    for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, n, torch.bfloat16, 3)
    _need(reserve, "reserve", torch.uint8, 1)
    T, H = x.shape
    E, F, _ = w_gate.shape
    dev = x.device
    nws = backward_workspace_bytes(T, H, F, E, k)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    if grads is None:
        grads = dict(dx=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
                     dw_router=torch.empty((E, H), dtype=torch.float32, device=dev),
                     dw_gate=torch.empty((E, F, H), dtype=torch.bfloat16, device=dev),
                     dw_up=torch.empty((E, F, H), dtype=torch.bfloat16, device=dev),
                     dw_down=torch.empty((E, H, F), dtype=torch.bfloat16, device=dev))
    lib, st = _lib.load(), _stream(dev)
    if split:
        check(lib.moe_layer_backward_data(
            _p(x), MOE_BF16, _p(w_router), _p(w_gate), _p(w_up), _p(w_down), MOE_BF16, T, H, F,
            E, k, _p(dout), _p(reserve), reserve.numel(), _p(grads["dx"]),
            _p(grads["dw_router"]), _p(workspace), workspace.numel(), st))
        check(lib.moe_layer_backward_weights(
            T, H, F, E, k, _p(reserve), reserve.numel(), _p(grads["dw_gate"]), _p(grads["dw_up"]),
            _p(grads["dw_down"]), _p(workspace), workspace.numel(), st))
        return grads
    check(lib.moe_layer_backward(
        _p(x), MOE_BF16, _p(w_router), _p(w_gate), _p(w_up), _p(w_down), MOE_BF16, T, H, F, E, k,
        _p(dout), _p(reserve), reserve.numel(), _p(grads["dx"]), _p(grads["dw_router"]),
        _p(grads["dw_gate"]), _p(grads["dw_up"]), _p(grads["dw_down"]), _p(workspace),
        workspace.numel(), st))
    return grads


def moe_layer_backward_weights(reserve: torch.Tensor, workspace: torch.Tensor, grads: dict,
                               T: int, H: int, F: int, E: int, k: int = 2):
    """The weight step alone (dw_gate, dw_up, dw_down into grads), reading
    what an earlier moe_layer_backward data step left in workspace."""
    _need(reserve, "reserve", torch.uint8, 1)
    _need(workspace, "workspace", torch.uint8, 1)
    for n in ("dw_gate", "dw_up", "dw_down"):
        _need(grads[n], n, torch.bfloat16, 3)
    check(_lib.load().moe_layer_backward_weights(
        T, H, F, E, k, _p(reserve), reserve.numel(), _p(grads["dw_gate"]), _p(grads["dw_up"]),
        _p(grads["dw_down"]), _p(workspace), workspace.numel(), _stream(reserve.device)))
    return grads
