"""GPU parity of moe_routing_stats (utilisation, margin to the next expert,
softmax mass outside the top k) against oracle.routing_stats.

Two sources of logits: seeded synthetic logits with many equal values (the
kernel and the oracle read the same float32 array, so results agree to the
last bit or within float32 rounding), and the router's own logits on the
parity and Grok-1-shape inputs (the oracle then uses its own float32 router
product, so margins and masses agree to the router's tolerance).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.device import generate_device
from gpu_helpers import check_routing, dev_tensor, host_array, log, to_device

pytestmark = pytest.mark.gpu

F32_ULP = 2.0 ** -23


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_transformer_top_amd as m
    m.load_library()
    return m


def compare(got, ref, margin_tol, mass_tol):
    g_m, g_s, g_u = (host_array(got[n]).astype(np.float64)
                     for n in ("margin", "unselected_mass", "utilization"))
    inf = np.isinf(ref.margin)
    assert np.array_equal(np.isinf(g_m), inf)
    assert np.all(np.abs(g_m[~inf] - ref.margin[~inf]) <= margin_tol(ref.margin[~inf]))
    assert np.all(np.abs(g_s - ref.unselected_mass) <= mass_tol(ref.unselected_mass))
    assert np.all(np.abs(g_u - ref.utilization) <= F32_ULP * np.abs(ref.utilization))


@pytest.mark.parametrize("T,E,k", [(0, 8, 2), (1, 8, 2), (300, 8, 2), (1000, 16, 4),
                                   (257, 4, 1), (50, 4, 4), (4099, 12, 3)])
def test_stats_on_synthetic_logits(moe, T, E, k):
    log(f"routing stats T={T} E={E} k={k}")
    l32 = synth.routing_logits(T, E, seed=T + 31 * E + k)
    counts = np.random.default_rng(T + E).integers(0, max(T, 1) * k + 1, E).astype(np.int32)
    got = moe.moe_routing_stats(dev_tensor(l32, "f32"), dev_tensor(counts, "i32"), k)
    torch.cuda.synchronize()
    ref = oracle.routing_stats(l32, k, counts)
    # the margin is one float32 subtraction of the same two values (correctly
    # rounded); the mass is float32 exp and sums over at most 16 terms
    compare(got, ref, lambda r: F32_ULP * np.abs(r),
            lambda r: 1e-6 + 1e-5 * r)


def test_stats_all_equal_logits(moe):
    # every logit equal: margin 0, mass (E - k) / E, for every token
    l32 = np.full((70, 8), 0.375, np.float32)
    got = moe.moe_routing_stats(dev_tensor(l32, "f32"), dev_tensor(np.full(8, 7, np.int32), "i32"), 2)
    torch.cuda.synchronize()
    assert np.all(host_array(got["margin"]) == 0.0)
    assert np.all(np.abs(host_array(got["unselected_mass"]) - 0.75) < 1e-7)
    assert np.all(host_array(got["utilization"]) == np.float32(7 * 8 / 140))


def _router_path(moe, x, wr, k, x64, wr_host):
    _, _, logits = moe.moe_router_topk(x, wr, k, return_logits=True)
    idx, w = moe.moe_router_topk(x, wr, k)
    disp = moe.moe_dispatch(idx, wr.shape[0], None)
    got = moe.moe_routing_stats(logits, disp["counts"], k)
    torch.cuda.synchronize()
    l32, l64 = oracle.router_logits(x64, wr_host)
    routing = oracle.top_k_softmax(l32, l64, k)
    ref = oracle.routing_stats(l32, k, oracle.dispatch(routing.idx, wr.shape[0], None).counts)
    diff = check_routing(host_array(idx), host_array(w), routing)
    scale = np.maximum(1.0, np.abs(l64).max(axis=1))
    return got, ref, diff, scale


@pytest.mark.parametrize("name", ["p_bf16", "p_skew", "p_f32", "p_dec1"])
def test_stats_on_router_logits(moe, name):
    cfg = synth.get_config(name)
    inp = synth.generate_host(cfg)
    d = to_device(inp)
    got, ref, diff, scale = _router_path(moe, d["x"], d["wr"], cfg.k,
                                         oracle.widen(inp.x, cfg.act), inp.wr)
    assert not diff.any()
    compare(got, ref, lambda r: 2e-5 * scale[~np.isinf(ref.margin)],
            lambda r: 1e-5 + 1e-4 * r)


@pytest.mark.parametrize("name", ["decode", "skew", "capacity"])
def test_stats_at_grok1_shape(moe, name):
    cfg = synth.CONFIGS[name]
    log(f"routing stats at {name}: T={cfg.T}")
    d = generate_device(cfg, "cuda", x_only=True)
    got, ref, diff, scale = _router_path(moe, d.x, d.wr, cfg.k,
                                         oracle.widen(host_array(d.x), cfg.act), host_array(d.wr))
    log(f"  tokens with a routing tie: {int(diff.sum())}")
    keep = ~diff
    g_m = host_array(got["margin"]).astype(np.float64)
    g_s = host_array(got["unselected_mass"]).astype(np.float64)
    assert np.all(np.abs(g_m - ref.margin)[keep] <= 2e-5 * scale[keep])
    assert np.all(np.abs(g_s - ref.unselected_mass)[keep] <= 1e-5 + 1e-4 * ref.unselected_mass[keep])
    if not diff.any():
        assert np.all(np.abs(host_array(got["utilization"]) - ref.utilization)
                      <= F32_ULP * ref.utilization)
    # the statistics the page talks about, for the log: mean margin and the
    # mass left outside the top 2
    log(f"  mean margin {g_m.mean():.3f}, mean outside mass {g_s.mean():.3f}, "
        f"utilisation {np.round(host_array(got['utilization']), 3).tolist()}")
    del d
    torch.cuda.empty_cache()
