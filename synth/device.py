"""Device-side seeded generation of Grok-1-shape layer inputs.

The Grok-1 shape holds 4.8e9 expert weights (9.66 GB in bf16); drawing them on
the host takes minutes, so they are drawn on the GPU with torch's Philox
generator. Each tensor gets its own seed, seed * 7919 + index, with index
0 = x, 1 = router W, 2 + 3e + {0, 1, 2} = W_gate[e], W_up[e], W_down[e].
Distributions, scales, storage rounding and the router skew are the same as in
the host generator (synth.gen). Only torch's own random and elementwise ops
run here; none of the layer's arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from .configs import LayerConfig


def _gen(device, seed: int, index: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 7919 + index)
    return g


def _randn(shape, std: float, device, seed: int, index: int) -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, 1.0, generator=_gen(device, seed, index))
    if std != 1.0:
        t.mul_(std)
    return t


def quantize_int8_rows_t(w: torch.Tensor):
    """Per-row absmax int8 quantisation (same rule as synth.gen.quantize_int8_rows)."""
    s = w.abs().amax(dim=1) / 127.0
    s_safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.round(w / s_safe[:, None]).clamp_(-127, 127).to(torch.int8)
    return q, s


def quantize_int4_groups_t(w: torch.Tensor, group: int = 128):
    """Group-wise symmetric int4 (same rule as synth.gen.quantize_int4_groups):
    packed unsigned nibbles q + 8, k even in the low nibble; scales [N, K/group]."""
    N, K = w.shape
    g = w.view(N, K // group, group)
    s = g.abs().amax(dim=2) / 7.0
    s_safe = torch.where(s > 0, s, torch.ones_like(s))
    u = (torch.round(g / s_safe[:, :, None]).clamp_(-7, 7) + 8).to(torch.uint8).view(N, K)
    return u[:, 0::2] | (u[:, 1::2] << 4), s


@dataclass
class DeviceInputs:
    cfg: LayerConfig
    x: torch.Tensor           # [T,H] float32 or bfloat16
    wr: torch.Tensor          # [E,H] float32
    wg: torch.Tensor          # [E,F,H]
    wu: torch.Tensor          # [E,F,H]
    wd: torch.Tensor          # [E,H,F]
    sg: Optional[torch.Tensor] = None
    su: Optional[torch.Tensor] = None
    sd: Optional[torch.Tensor] = None


def _store(w32: torch.Tensor, wdt: str):
    if wdt == "f32":
        return w32, None
    if wdt == "bf16":
        return w32.to(torch.bfloat16), None
    if wdt == "i8":
        return quantize_int8_rows_t(w32)
    if wdt == "i4":
        return quantize_int4_groups_t(w32)
    raise ValueError(wdt)


def generate_device(cfg: LayerConfig, device="cuda", seed: Optional[int] = None,
                    x_only: bool = False) -> DeviceInputs:
    seed = cfg.seed if seed is None else seed
    T, H, F, E = cfg.T, cfg.H, cfg.F, cfg.E
    x32 = _randn((T, H), 1.0, device, seed, 0)
    x = x32.to(torch.bfloat16) if cfg.act == "bf16" else x32
    del x32
    wr = _randn((E, H), H ** -0.5, device, seed, 1)
    if cfg.skew:
        m = x.to(torch.float64).mean(dim=0)
        u = (m / m.norm()).to(torch.float32)
        for e, a in enumerate(cfg.skew):
            wr[e] += torch.tensor(a, dtype=torch.float32, device=device) * u
    if x_only:
        return DeviceInputs(cfg, x, wr, None, None, None)

    wt = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8,
          "i4": torch.uint8}[cfg.wdt]
    half = 2 if cfg.wdt == "i4" else 1
    wg = torch.empty((E, F, H // half), dtype=wt, device=device)
    wu = torch.empty((E, F, H // half), dtype=wt, device=device)
    wd = torch.empty((E, H, F // half), dtype=wt, device=device)
    sg = su = sd = None
    f32 = dict(dtype=torch.float32, device=device)
    if cfg.wdt == "i8":
        sg, su, sd = torch.empty((E, F), **f32), torch.empty((E, F), **f32), torch.empty((E, H), **f32)
    if cfg.wdt == "i4":
        sg, su = torch.empty((E, F, H // 128), **f32), torch.empty((E, F, H // 128), **f32)
        sd = torch.empty((E, H, F // 128), **f32)
    for e in range(E):
        for j, (dst, shape, std, sdst) in enumerate((
                (wg, (F, H), H ** -0.5, sg),
                (wu, (F, H), H ** -0.5, su),
                (wd, (H, F), F ** -0.5, sd))):
            w32 = _randn(shape, std, device, seed, 2 + 3 * e + j)
            q, s = _store(w32, cfg.wdt)
            dst[e].copy_(q)
            if s is not None:
                sdst[e].copy_(s)
            del w32, q
    return DeviceInputs(cfg, x, wr, wg, wu, wd, sg, su, sd)


def grad_output_device(T: int, H: int, seed: int, device="cuda") -> torch.Tensor:
    """Seeded gradient of the layer output [T,H] ~ N(0,1) in bf16 (index 10^6
    keeps its stream apart from the layer inputs')."""
    return _randn((T, H), 1.0, device, seed, 1_000_000).to(torch.bfloat16)
