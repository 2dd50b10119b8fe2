"""Seeded synthetic inputs for the top-2 MoE FFN layer.

This module is shared by the oracle side and the GPU side of every test and
benchmark. It holds only input construction: Gaussian draws, the rounding of
draws to the storage dtype (bf16 round-to-nearest-even, int8 absmax
quantisation) and the router-skew construction. It contains none of the
layer's arithmetic (no router product, no top-k, no dispatch, no expert FFN).

Shapes follow the layer as described on the n4n.ai page "How does Grok-1 use a
mixture-of-experts design?" (section "The high-level architecture": hidden
6144, expert dim 32768, 8 experts, top-2; section "Expert implementation:
SwiGLU at scale" for the expert weight shapes, stored as nn.Linear [out, in]).
"""
from .configs import LayerConfig, CONFIGS, PARITY_CONFIGS, get_config  # noqa: F401
from .gen import (  # noqa: F401
    routing_logits,
    grad_output,
    HostInputs,
    generate_host,
    router_inputs,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    quantize_int8_rows,
    quantize_int4_groups,
    INT4_GROUP,
)
