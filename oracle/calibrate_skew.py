"""Calibrate the router-skew magnitudes of the skewed workloads.

The skewed workloads add a0 * u to router row 0 and a1 * u to row 1, u the
unit vector along the column mean of x. This script searches (a0, a1) so that
the oracle's top-1 pick lands on expert 0 for about 50% of the tokens and on
expert 1 for about 25%, at the given token count (H = 6144, seed 0 draws from
synth.gen). It prints the chosen magnitudes and the shares they give; the
values are then written into synth/configs.py by hand.

    python -m oracle.calibrate_skew --T 4096
"""
import argparse
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
from synth.gen import bf16_bits_from_f32, f32_from_bf16_bits, skew_direction  # noqa: E402


def shares(x64, wr, u, a0, a1):
    w = wr.copy()
    w[0] += np.float32(a0) * u
    w[1] += np.float32(a1) * u
    l32, l64 = oracle.router_logits(x64, w)
    top1 = oracle.top_k_softmax(l32, l64, 2).idx[:, 0]
    return np.mean(top1 == 0), np.mean(top1 == 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--T", type=int, required=True)
    ap.add_argument("--H", type=int, default=6144)
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    rng = np.random.Generator(np.random.PCG64(args.seed))
    x = f32_from_bf16_bits(bf16_bits_from_f32(
        rng.standard_normal((args.T, args.H), dtype=np.float32)))
    wr = (rng.standard_normal((8, args.H), dtype=np.float32) / np.sqrt(args.H)).astype(np.float32)
    u = skew_direction(x)
    x64 = x.astype(np.float64)
    best = None
    grid0 = np.arange(0.0, 8.01, 0.2)
    for a0 in grid0:
        for a1 in np.arange(0.0, a0 + 1e-9, 0.2):
            s0, s1 = shares(x64, wr, u, a0, a1)
            d = (s0 - 0.5) ** 2 + (s1 - 0.25) ** 2
            if best is None or d < best[0]:
                best = (d, round(float(a0), 2), round(float(a1), 2), s0, s1)
    _, a0, a1, s0, s1 = best
    print(f"T={args.T}: a0={a0} a1={a1} top1 shares expert0={s0:.4f} expert1={s1:.4f}")


if __name__ == "__main__":
    main()
