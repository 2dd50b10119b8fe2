"""GPU parity over a seeded sweep of layer shapes drawn at random: expert
counts 1 … 16, k up to 4, token counts on both sides of the decode/tiled
boundary (int4 weights: decode sizes only, as the library supports),
hidden and expert sizes that are multiples of 64 but not of the
256-wide tiles, every weight type, capacity factors that drop and that do
not, skewed and plain routers. Each case runs the whole layer and compares
routing, dispatch and output with the oracle, as test_gpu_shapes does for
its hand-picked cases."""
import numpy as np
import pytest

import synth
from gpu_helpers import check_close, check_routing, host_array, log, out_as_f64, to_device
from test_gpu_shapes import run_layer

pytestmark = pytest.mark.gpu


def _draw_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        E = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
        k = int(rng.integers(1, min(E, 4) + 1))
        T = int(rng.integers(1, 17)) if c % 3 == 0 else int(rng.integers(17, 700))
        wdt = str(rng.choice(["bf16", "bf16", "i8", "i4", "f32"]))
        if wdt == "i4":   # int4 weights run on the decode kernels only (T <= 16)
            T = int(rng.integers(1, 17))
        step = 128 if wdt == "i4" else 64
        H = step * int(rng.integers(1, 640 // step + 1))
        F = step * int(rng.integers(1, 768 // step + 1))
        act = "f32" if wdt == "f32" else "bf16"
        cf = [None, 0.5, 1.0, 1.25, 2.0][int(rng.integers(0, 5))]
        skew = (float(rng.uniform(1, 3)), float(rng.uniform(0.5, 2))) if rng.random() < 0.3 else ()
        cases.append(synth.LayerConfig(f"r{c}_E{E}k{k}T{T}H{H}F{F}{wdt}", T=T, H=H, F=F, E=E, k=k,
                                       act=act, wdt=wdt, capacity_factor=cf, skew=skew,
                                       seed=1000 + c))
    return cases


CASES = _draw_cases()


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_transformer_top_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_random_layer_shape(moe, cfg):
    log(f"random shape {cfg.name} cf={cfg.capacity_factor} skew={cfg.skew}")
    inp = synth.generate_host(cfg)
    out, ax, res = run_layer(moe, cfg, inp, to_device(inp))
    diff = check_routing(host_array(ax["topk_idx"]), host_array(ax["topk_w"]), res.routing)
    assert not diff.any()
    assert np.array_equal(host_array(ax["counts"]), res.disp.counts)
    assert np.array_equal(host_array(ax["offsets"]), res.disp.offsets)
    assert np.array_equal(host_array(ax["dropped"]), res.disp.dropped)
    check_close(out_as_f64(out), res.out, cfg.act, cfg.name)
