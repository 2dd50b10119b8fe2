"""Workload configurations of the MoE FFN layer.

Grok-1 shape: hidden H = 6144, expert dim F = 32768, E = 8 experts, top-k = 2
(n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section "The
high-level architecture", GrokMoELayer constructor). The capacity factor 1.25
and "capacity = factor x mean load" come from the section "Routing: top-2
without auxiliary loss"; the mean load per expert T*k/E from the section
"Tradeoffs: when MoE wins and when it doesn't" (expert batch size analysis).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                      # tokens (batch * seq_len, flattened)
    H: int                      # hidden size
    F: int                      # expert dim
    E: int = 8                  # experts
    k: int = 2                  # experts per token
    capacity_factor: Optional[float] = None   # None: no capacity limit
    act: str = "bf16"           # activation storage dtype: "f32" | "bf16"
    wdt: str = "bf16"           # expert weight storage dtype: "f32" | "bf16" | "i8" | "i4"
    # Router skew: row e of the router weight gets skew[e] * u added, with u
    # the unit vector along the mean of the (stored) token activations.
    skew: Tuple[float, ...] = field(default_factory=tuple)
    seed: int = 0
    description: str = ""

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    @property
    def n_assign(self) -> int:
        return self.T * self.k

    def expert_weight_bytes(self) -> int:
        """Bytes of one expert's three matrices at the storage dtype."""
        if self.wdt == "i4":   # packed nibbles + one float32 scale per 128 k
            return 3 * self.H * self.F // 2 + 3 * self.H * self.F // 128 * 4
        per = {"f32": 4, "bf16": 2, "i8": 1}[self.wdt]
        return 3 * self.H * self.F * per


# Skew magnitudes. The literal reading "+0.5 / +0.25 of the mean direction"
# moves only about a quarter / a sixth of the top-1 picks onto experts 0 / 1,
# so the magnitudes were chosen by a search on a 0.2 grid (host draws, seed 0)
# to put roughly 50% and 25% of the top-1 picks on experts 0 and 1 at each
# token count: 50.3% / 24.6% at T = 4096, and at T = 16384 the closest the grid
# reached, 47.1% / 22.6% (tests/test_synth.py pins both).
SKEW_T4096 = (1.8, 1.4)
SKEW_T16384 = (8.0, 7.4)

CONFIGS = {
    "tiny": LayerConfig(
        "tiny", T=32, H=128, F=512, act="f32", wdt="f32",
        description="tiny fp32 top-2 layer: T=32, H=128, F=512, no capacity"),
    "decode": LayerConfig(
        "decode", T=8, H=6144, F=32768,
        description="Grok-1 shape decode: T=8, bf16, fp32 router, no drop"),
    "prefill": LayerConfig(
        "prefill", T=8192, H=6144, F=32768,
        description="Grok-1 shape prefill: one 8192-token context, bf16, no drop"),
    "skew": LayerConfig(
        "skew", T=4096, H=6144, F=32768, skew=SKEW_T4096,
        description="skewed routing, T=4096, bf16"),
    "capacity": LayerConfig(
        "capacity", T=16384, H=6144, F=32768, capacity_factor=1.25,
        wdt="i8", skew=SKEW_T16384,
        description="capacity 1.25, int8 weights with per-row fp32 scales, skewed router, T=16384"),
    "train": LayerConfig(
        "train", T=8192, H=6144, F=32768, capacity_factor=1.25,
        description="Grok-1 shape training step (forward keeping activations + backward): "
                    "one 8192-token batch, bf16, capacity 1.25"),
    "medium": LayerConfig(
        "medium", T=512, H=6144, F=32768,
        description="Grok-1 shape medium batch: one 512-token sequence (about 128 rows per "
                    "expert), bf16, no drop"),
    "decode_i4": LayerConfig(
        "decode_i4", T=8, H=6144, F=32768, wdt="i4",
        description="Grok-1 shape decode with int4 weights (one fp32 scale per row and 128 k): "
                    "T=8, bf16 activations, no drop"),
}

# Sizes small enough for an element-by-element comparison with the oracle
# that still span several GEMM tiles and leave ragged per-expert tails.
PARITY_CONFIGS = {
    "p_f32": LayerConfig("p_f32", T=77, H=256, F=384, act="f32", wdt="f32", seed=3),
    "p_bf16": LayerConfig("p_bf16", T=301, H=512, F=768, seed=4),
    "p_bf16_dec": LayerConfig("p_bf16_dec", T=13, H=1024, F=2048, seed=5),
    "p_i8": LayerConfig("p_i8", T=190, H=512, F=1024, wdt="i8", seed=6),
    "p_cap": LayerConfig("p_cap", T=517, H=256, F=512, capacity_factor=1.25,
                         skew=(1.8, 1.4), seed=7),
    "p_cap_i8": LayerConfig("p_cap_i8", T=260, H=256, F=512, capacity_factor=1.25,
                            wdt="i8", skew=(2.5, 2.0), seed=8),
    "p_skew": LayerConfig("p_skew", T=640, H=512, F=512, skew=(1.8, 1.4), seed=9),
    # column counts that are not multiples of the GEMM tile widths
    "p_bf16_tail": LayerConfig("p_bf16_tail", T=150, H=320, F=448, seed=10),
    "p_i8_dec": LayerConfig("p_i8_dec", T=9, H=512, F=1024, wdt="i8", seed=11),
    "p_dec1": LayerConfig("p_dec1", T=1, H=384, F=640, seed=12),
    "p_i4_dec": LayerConfig("p_i4_dec", T=9, H=512, F=1024, wdt="i4", seed=13),
    "p_i4_dec16": LayerConfig("p_i4_dec16", T=16, H=640, F=384, wdt="i4", seed=14),
    "p_i4_dec1": LayerConfig("p_i4_dec1", T=1, H=384, F=640, wdt="i4", seed=15),
}


def get_config(name: str) -> LayerConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in PARITY_CONFIGS:
        return PARITY_CONFIGS[name]
    raise KeyError(name)
