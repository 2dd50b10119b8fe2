"""Host-side seeded generation (numpy PCG64) of layer inputs.

Draw order, all from one numpy Generator(PCG64(seed)):
  x [T,H] ~ N(0,1); router W [E,H] ~ N(0,1/H); then for e = 0..E-1:
  W_gate[e] [F,H] ~ N(0,1/H), W_up[e] [F,H] ~ N(0,1/H), W_down[e] [H,F] ~ N(0,1/F).
Draws are float32. Storage conversions:
  bf16 : round-to-nearest-even of the float32 draw, kept as uint16 bit patterns;
  i8   : per output row, s = max|w| / 127 and q = clip(rint(w / s), -127, 127).
The router weight always stays float32. A skewed router adds skew[e] * u to
row e, u the unit vector along the column mean of x as stored.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from .configs import LayerConfig


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs are finite (no NaN handling is needed for Gaussian draws)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def quantize_int8_rows(w: np.ndarray):
    """Per-output-row absmax int8 quantisation of a float32 matrix [N, K].

    Returns (q int8 [N,K], s float32 [N]) with w ~= q * s[:, None]."""
    w = np.asarray(w, dtype=np.float32)
    s = (np.max(np.abs(w), axis=1) / np.float32(127.0)).astype(np.float32)
    s_safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(w / s_safe[:, None]), -127, 127).astype(np.int8)
    return q, s


INT4_GROUP = 128   # k values sharing one int4 scale


def quantize_int4_groups(w: np.ndarray):
    """Symmetric int4 quantisation of a float32 matrix [N, K] with one scale
    per row and group of 128 consecutive k: s = max|w| / 7 over the group,
    q = clip(rint(w / s), -7, 7). Stored as unsigned nibbles u = q + 8, two
    per byte (k even in the low nibble).

    Returns (packed uint8 [N, K/2], s float32 [N, K/128]) with
    w ~= (u - 8) * s."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    g = w.reshape(N, K // INT4_GROUP, INT4_GROUP)
    s = (np.max(np.abs(g), axis=2) / np.float32(7.0)).astype(np.float32)
    s_safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(g / s_safe[:, :, None]), -7, 7).astype(np.int16).reshape(N, K)
    u = (q + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << np.uint8(4))).astype(np.uint8), s


@dataclass
class HostInputs:
    """Arrays of one layer instance as the layer stores them.

    x   : float32 [T,H] (act f32) or uint16 bf16 bits [T,H] (act bf16)
    wr  : float32 [E,H]
    wg, wu : [E,F,H]; wd : [E,H,F]  -- float32, uint16 bf16 bits, or int8;
             int4: packed uint8 [E,F,H/2] and [E,H,F/2]
    sg, su : float32 [E,F]; sd : float32 [E,H]  -- int8 row scales; int4:
             [E,F,H/128] and [E,H,F/128] group scales
    """
    cfg: LayerConfig
    x: np.ndarray
    wr: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    sg: Optional[np.ndarray] = None
    su: Optional[np.ndarray] = None
    sd: Optional[np.ndarray] = None

    def arrays(self) -> Dict[str, np.ndarray]:
        d = dict(x=self.x, wr=self.wr, wg=self.wg, wu=self.wu, wd=self.wd)
        if self.sg is not None:
            d.update(sg=self.sg, su=self.su, sd=self.sd)
        return d


def _store_weight(w32: np.ndarray, wdt: str):
    if wdt == "f32":
        return w32, None
    if wdt == "bf16":
        return bf16_bits_from_f32(w32), None
    if wdt == "i8":
        return quantize_int8_rows(w32)
    if wdt == "i4":
        return quantize_int4_groups(w32)
    raise ValueError(wdt)


def x_as_f32(x: np.ndarray, act: str) -> np.ndarray:
    return f32_from_bf16_bits(x) if act == "bf16" else np.asarray(x, np.float32)


def skew_direction(x_stored_f32: np.ndarray) -> np.ndarray:
    """Unit vector (float32) along the column mean of the activations."""
    m = x_stored_f32.astype(np.float64).mean(axis=0)
    n = np.linalg.norm(m)
    return (m / n).astype(np.float32) if n > 0 else np.zeros_like(m, np.float32)


def _draw_router_inputs(rng, cfg: LayerConfig):
    """The first two draws of a layer instance: x (stored form) and the router
    weight before the skew."""
    T, H, E = cfg.T, cfg.H, cfg.E
    f32 = np.float32
    x32 = rng.standard_normal((T, H), dtype=f32)
    wr = (rng.standard_normal((E, H), dtype=f32) * f32(1.0 / np.sqrt(H))).astype(f32)
    x = bf16_bits_from_f32(x32) if cfg.act == "bf16" else x32
    return x, wr


def _apply_skew(x, wr, cfg: LayerConfig):
    if cfg.skew:
        u = skew_direction(x_as_f32(x, cfg.act))
        for e, a in enumerate(cfg.skew):
            wr[e] = (wr[e] + np.float32(a) * u).astype(np.float32)
    return wr


def router_inputs(cfg: LayerConfig, seed: Optional[int] = None):
    """x and the router weight (skew applied) exactly as generate_host draws
    them, without drawing the expert weights."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    x, wr = _draw_router_inputs(rng, cfg)
    return x, _apply_skew(x, wr, cfg)


def generate_host(cfg: LayerConfig, seed: Optional[int] = None) -> HostInputs:
    """Draw one layer instance on the host (sizes up to a few hundred MB)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    T, H, F, E = cfg.T, cfg.H, cfg.F, cfg.E
    f32 = np.float32
    x, wr = _draw_router_inputs(rng, cfg)

    wdt_np = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8, "i4": np.uint8}[cfg.wdt]
    half = 2 if cfg.wdt == "i4" else 1
    wg = np.empty((E, F, H // half), wdt_np)
    wu = np.empty((E, F, H // half), wdt_np)
    wd = np.empty((E, H, F // half), wdt_np)
    sg = su = sd = None
    if cfg.wdt == "i8":
        sg = np.empty((E, F), f32)
        su = np.empty((E, F), f32)
        sd = np.empty((E, H), f32)
    if cfg.wdt == "i4":
        sg = np.empty((E, F, H // INT4_GROUP), f32)
        su = np.empty((E, F, H // INT4_GROUP), f32)
        sd = np.empty((E, H, F // INT4_GROUP), f32)
    for e in range(E):
        g = rng.standard_normal((F, H), dtype=f32) * f32(1.0 / np.sqrt(H))
        u = rng.standard_normal((F, H), dtype=f32) * f32(1.0 / np.sqrt(H))
        d = rng.standard_normal((H, F), dtype=f32) * f32(1.0 / np.sqrt(F))
        wg[e], s0 = _store_weight(g.astype(f32), cfg.wdt)
        wu[e], s1 = _store_weight(u.astype(f32), cfg.wdt)
        wd[e], s2 = _store_weight(d.astype(f32), cfg.wdt)
        if cfg.wdt in ("i8", "i4"):
            sg[e], su[e], sd[e] = s0, s1, s2

    wr = _apply_skew(x, wr, cfg)
    return HostInputs(cfg, x, wr, wg, wu, wd, sg, su, sd)


def routing_logits(T: int, E: int, seed: int, tie_frac: float = 0.3) -> np.ndarray:
    """Seeded float32 logits [T,E]: N(0,1) draws with a fraction of entries
    replaced by small integers, so that equal values (also at the k / k+1
    boundary) occur."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((T, E))
    ints = rng.integers(-2, 3, (T, E)).astype(np.float64)
    return np.where(rng.random((T, E)) < tie_frac, ints, g).astype(np.float32)



def grad_output(T: int, H: int, seed: int) -> np.ndarray:
    """Seeded gradient of the layer output [T,H] ~ N(0,1), as bf16 bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))
