"""Top-2 mixture-of-experts FFN layer (Grok-1 shape) for AMD MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe.so, built in-tree by sparse_moe_transformer_top_amd.build); this
package is its Python binding. The library is loaded at the first call and
its absence raises ImportError (there is no fallback path).
"""
from .api import (  # noqa: F401
    backward_workspace_bytes,
    layer_workspace_bytes,
    moe_combine,
    moe_dispatch,
    moe_ep_pack,
    moe_ep_recv_layout,
    moe_ep_unpack,
    moe_expert_down,
    moe_expert_ffn,
    moe_expert_gate_up,
    moe_layer_backward,
    moe_layer_backward_weights,
    moe_layer_forward,
    moe_layer_forward_noalloc,
    moe_layer_forward_train,
    moe_router_topk,
    moe_routing_stats,
    train_reserve_bytes,
    train_reserve_views,
)
from ._lib import MoeError, LIB_PATH, NOALLOC_SCRATCH_BYTES, load as load_library  # noqa: F401
