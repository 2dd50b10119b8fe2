"""GPU parity at the Grok-1 shape (H = 6144, F = 32768, E = 8, k = 2) in the
launch configuration bench.py times (moe_layer_forward on device-generated
inputs).

Routing and dispatch are compared for every token; the layer output on a
seeded sample of 256 tokens (all tokens for decode), which the oracle
evaluates one by one in float64. Inputs come from synth.device (torch Philox
draws on the GPU); the oracle reads host copies of exactly those arrays.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.device import generate_device
from gpu_helpers import (LazyExperts, check_close, check_dispatch_equal, check_weights,
                         gpu_routing, host_array, log, out_as_f64)

pytestmark = pytest.mark.gpu

_weights = {}


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_transformer_top_amd as m
    m.load_library()
    yield m
    _weights.clear()
    torch.cuda.empty_cache()


# medium batches at the Grok-1 H and F (the page's batch = 1, seq = 512 point
# and two smaller ones): 16 to 128 rows per expert
MEDIUM = {f"t{T}": synth.CONFIGS["medium"].with_(name=f"t{T}", T=T, seed=70 + T)
          for T in (64, 128)}


def inputs(name):
    cfg = synth.CONFIGS[name] if name in synth.CONFIGS else MEDIUM[name]
    # bf16 workloads share one weight set (same seed): draw it once
    if cfg.wdt == "bf16":
        if "bf16" not in _weights:
            _weights.clear()
            torch.cuda.empty_cache()
            _weights["bf16"] = generate_device(cfg, "cuda")
        w = _weights["bf16"]
        xd = generate_device(cfg, "cuda", x_only=True)
        return cfg, type(w)(cfg, xd.x, xd.wr, w.wg, w.wu, w.wd)
    _weights.clear()
    torch.cuda.empty_cache()
    return cfg, generate_device(cfg, "cuda")


@pytest.mark.parametrize("name", ["decode", "t64", "t128", "medium", "prefill", "skew",
                                  "capacity", "decode_i4"])
def test_fullsize_layer(moe, name):
    cfg, d = inputs(name)
    _check_layer(moe, cfg, d, name)


@pytest.mark.parametrize("wdt", ["bf16", "i8"])
def test_x_beyond_2gib(moe, wdt):
    # x larger than 2 GiB (180 000 tokens of 6144): the gate/up kernel
    # addresses the gathered rows with 64-bit per-lane pointers instead of
    # 32-bit offsets from x; a small F keeps h and the weights small
    cfg = synth.LayerConfig("x_wide_" + wdt, T=180_000, H=6144, F=128, wdt=wdt, seed=51)
    assert cfg.T * cfg.H * 2 > 2 ** 31
    _weights.clear()
    torch.cuda.empty_cache()
    d = generate_device(cfg, "cuda")
    _check_layer(moe, cfg, d, cfg.name)
    del d
    torch.cuda.empty_cache()


def _check_layer(moe, cfg, d, name):
    log(f"full-size {name}: T={cfg.T} {cfg.act}/{cfg.wdt} cf={cfg.capacity_factor}")
    out, ax = moe.moe_layer_forward(d.x, d.wr, d.wg, d.wu, d.wd, k=cfg.k,
                                    capacity_factor=cfg.capacity_factor, s_gate=d.sg,
                                    s_up=d.su, s_down=d.sd, aux=True)
    torch.cuda.synchronize()
    T = cfg.T
    sample = np.arange(T) if T <= 256 else np.sort(
        np.random.default_rng(1).choice(T, 256, replace=False))
    sc = {n: (None if getattr(d, n) is None else host_array(getattr(d, n)))
          for n in ("sg", "su", "sd")}
    x_h, wr_h = host_array(d.x), host_array(d.wr)
    # routing of every token against the oracle's; the reference then uses
    # the GPU's own choice where a tie-flagged token was ordered differently
    l32, l64 = oracle.router_logits(oracle.widen(x_h, cfg.act), wr_h)
    routing = oracle.top_k_softmax(l32, l64, cfg.k)
    idx, w = host_array(ax["topk_idx"]), host_array(ax["topk_w"])
    own = gpu_routing(idx, w, routing)
    log(f"  tie-flagged tokens {int(routing.tie.sum())}; oracle on {len(sample)} tokens")
    res = oracle.layer_forward(x_h, cfg.act, wr_h, LazyExperts(d.wg), LazyExperts(d.wu),
                               LazyExperts(d.wd), cfg.wdt, k=cfg.k,
                               capacity_factor=cfg.capacity_factor, sg=sc["sg"], su=sc["su"],
                               sd=sc["sd"], tokens=sample, idx=own)
    check_weights(w, res.routing)
    # dispatch of all T*k assignments, bit-exact: the layer's counts, offsets
    # and drops, and perm / slot_row of the dispatch of the layer's indices
    assert np.array_equal(host_array(ax["counts"]), res.disp.counts)
    assert np.array_equal(host_array(ax["offsets"]), res.disp.offsets)
    assert np.array_equal(host_array(ax["dropped"]), res.disp.dropped)
    got = moe.moe_dispatch(ax["topk_idx"], cfg.E, cfg.capacity_factor)
    torch.cuda.synchronize()
    check_dispatch_equal({k: host_array(v) for k, v in got.items()}, res.disp)
    r = check_close(out_as_f64(out)[sample], res.out, cfg.act, f"{name} out")
    log(f"  out: max ratio {r[0]:.2e}, l2 ratio {r[1]:.2e}")
    if cfg.capacity_factor is not None:
        assert res.disp.cap == 5120
        assert int(res.disp.dropped.sum()) > 0
        log(f"  kept {int(res.disp.offsets[-1])} of {T * cfg.k} assignments")
    if cfg.skew:
        top1 = np.bincount(idx[:, 0], minlength=cfg.E) / T
        log(f"  top-1 shares {np.round(top1, 3).tolist()}")
        assert top1[0] > 0.3 and top1[1] > 0.15
