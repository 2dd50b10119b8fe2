"""ctypes loader and signatures of libmoe.so (the C ABI in include/moe.h).

torch is imported first so that the HIP runtime torch loaded is the one the
library binds to (one libamdhip64 per process; stream handles from torch are
only valid in that runtime). A missing library is an ImportError: there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # noqa: F401  (loads the HIP runtime first)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_F32, MOE_BF16, MOE_I8, MOE_I4 = 0, 1, 2, 3

# MOE_NOALLOC_SCRATCH_BYTES: the fixed workspace of moe_layer_forward_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20

# exported symbols and their (restype, argtypes)
_P, _I32, _I64, _F, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
SIGNATURES = {
    "moe_status_string": (C.c_char_p, [C.c_int]),
    "moe_last_error": (C.c_char_p, []),
    "moe_router_topk": (C.c_int, [_P, C.c_int, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P]),
    "moe_dispatch_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "moe_dispatch": (C.c_int, [_P, _I64, _I32, _I32, _F, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32, C.c_int, C.c_int]),
    "moe_expert_ffn": (C.c_int, [_P, C.c_int, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P,
                                 C.c_int, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_gate_up": (C.c_int, [_P, C.c_int, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P,
                                     C.c_int, _P, _P, _P, _P]),
    "moe_expert_down": (C.c_int, [_P, C.c_int, _P, _I64, _I32, _I32, _I32, _I32, _P, C.c_int,
                                  _P, _P, _P, _SZ, _P]),
    "moe_combine": (C.c_int, [_P, _P, _P, _I64, _I32, _I32, C.c_int, _P, _P]),
    "moe_routing_stats": (C.c_int, [_P, _P, _I64, _I32, _I32, _P, _P, _P, _P]),
    "moe_ep_pack": (C.c_int, [_P, C.c_int, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "moe_ep_recv_layout": (C.c_int, [_P, _I32, _I32, _I64, _P, _P, _P]),
    "moe_ep_unpack": (C.c_int, [_P, C.c_int, _P, _P, _I32, _I32, _I64, _P, _P]),
    "moe_layer_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32, C.c_int, C.c_int]),
    "moe_layer_forward": (C.c_int, [_P, C.c_int, _P, _P, _P, _P, C.c_int, _P, _P, _P, _I64, _I32,
                                    _I32, _I32, _I32, _F, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_forward_noalloc": (C.c_int, [_P, C.c_int, _P, _P, _P, _P, C.c_int, _P, _P, _P,
                                            _I64, _I32, _I32, _I32, _I32, _F, _P, _P, _P, _P, _P,
                                            _P, _P]),
    "moe_layer_train_reserve_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32]),
    "moe_layer_backward_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32]),
    "moe_layer_forward_train": (C.c_int, [_P, C.c_int, _P, _P, _P, _P, C.c_int, _I64, _I32, _I32,
                                          _I32, _I32, _F, _P, _P, _SZ, _P]),
    "moe_layer_backward": (C.c_int, [_P, C.c_int, _P, _P, _P, _P, C.c_int, _I64, _I32, _I32, _I32,
                                     _I32, _P, _P, _SZ, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_backward_data": (C.c_int, [_P, C.c_int, _P, _P, _P, _P, C.c_int, _I64, _I32, _I32,
                                          _I32, _I32, _P, _P, _SZ, _P, _P, _P, _SZ, _P]),
    "moe_layer_backward_weights": (C.c_int, [_I64, _I32, _I32, _I32, _I32, _P, _SZ, _P, _P, _P,
                                             _P, _SZ, _P]),
}

_lib = None


def load() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_moe_transformer_top_amd.build` (hipcc, gfx950)")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


def status_string(s: int) -> str:
    return load().moe_status_string(s).decode()


def check(status: int):
    if status != MOE_OK:
        raise MoeError(status, load().moe_last_error().decode())
