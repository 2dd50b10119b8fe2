"""GPU parity of every step of the layer against the oracle (through the C ABI).

Sizes here run the oracle element by element in seconds and still span
several GEMM tiles, ragged per-expert tails and column tails; the decode
kernels (T <= 16) and the tiled kernels (T > 16) are both covered, in bf16,
int8 and float32, with and without capacity drops, and int4 on the decode
kernels.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (check_close, check_dispatch_equal, check_routing, check_weights,
                         dev_tensor, gpu_routing, host_array, log, out_as_f64, to_device)

pytestmark = pytest.mark.gpu

ALL = ["tiny", "p_f32", "p_bf16", "p_bf16_dec", "p_i8", "p_cap", "p_cap_i8", "p_skew",
       "p_bf16_tail", "p_i8_dec", "p_dec1", "p_i4_dec", "p_i4_dec16", "p_i4_dec1"]


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_transformer_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


_cache = {}


def case(name):
    """(cfg, host inputs, device inputs, oracle full-layer result) per config."""
    if name not in _cache:
        cfg = synth.get_config(name)
        inp = synth.generate_host(cfg)
        res = oracle.layer_forward(inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt,
                                   k=cfg.k, capacity_factor=cfg.capacity_factor,
                                   sg=inp.sg, su=inp.su, sd=inp.sd)
        _cache[name] = (cfg, inp, to_device(inp), res)
    return _cache[name]


@pytest.mark.parametrize("name", ALL)
def test_router_topk(moe, name):
    cfg, inp, d, res = case(name)
    log(f"router {name} T={cfg.T} H={cfg.H}")
    idx, w, logits = moe.moe_router_topk(d["x"], d["wr"], cfg.k, return_logits=True)
    torch.cuda.synchronize()
    lg = host_array(logits).astype(np.float64)
    scale = np.maximum(1.0, np.abs(res.routing.l64).max(axis=1, keepdims=True))
    assert np.max(np.abs(lg - res.routing.l64) / scale) < 2e-5
    check_routing(host_array(idx), host_array(w), res.routing)


# Many tokens: the matrix-core router (bf16 x, E <= 8, from 4608 tokens).
# Cases: the Grok-1 prefill shape; a ragged last group of 32 tokens; hidden
# sizes whose 64-wide chunks split unevenly over the 4 waves (7 chunks: 2, 2,
# 2, 1; 17 chunks) or leave waves without a chunk (H = 64); E = 6, 4, 2, 1
# with k = 3, 1, 4, 2, 1 (E = k: every expert selected; E = 1: the weight is
# 1); and the vector kernel at the same token counts (float32 x, E > 8) and
# just below the threshold.
ROUTER_MANY = [
    # name, T, H, E, k
    ("grok_prefill", 8192, 6144, 8, 2),
    ("ragged", 4608 + 17, 512, 8, 2),
    ("h448_e6_k3", 5001, 448, 6, 3),
    ("h64_e4_k1", 4650, 64, 4, 1),
    ("h1088_k4", 6000, 1088, 8, 4),
    ("f32_vector", 4608, 256, 8, 2),
    ("e12_vector", 4608, 256, 12, 2),
    ("below_threshold", 4607, 512, 8, 2),
    ("at_threshold_e2_k2", 4608, 320, 2, 2),
    ("e1_k1", 4609, 128, 1, 1),
]


@pytest.mark.parametrize("name,T,H,E,k", ROUTER_MANY, ids=[r[0] for r in ROUTER_MANY])
def test_router_topk_many_tokens(moe, name, T, H, E, k):
    cfg = synth.LayerConfig(f"router_{name}", T=T, H=H, F=64, E=E, k=k, seed=200 + T % 97,
                            act="f32" if name.startswith("f32") else "bf16")
    inp = synth.generate_host(cfg)
    log(f"router {name} T={T} H={H} E={E} k={k}")
    x64 = oracle.widen(inp.x, cfg.act)
    l32, l64 = oracle.router_logits(x64, inp.wr)
    routing = oracle.top_k_softmax(l32, l64, k)
    d = to_device(inp)
    idx, w, logits = moe.moe_router_topk(d["x"], d["wr"], k, return_logits=True)
    torch.cuda.synchronize()
    lg = host_array(logits).astype(np.float64)
    scale = np.maximum(1.0, np.abs(l64).max(axis=1, keepdims=True))
    assert np.max(np.abs(lg - l64) / scale) < 2e-5
    check_routing(host_array(idx), host_array(w), routing)


@pytest.mark.parametrize("name", ALL)
def test_dispatch_on_oracle_indices(moe, name):
    cfg, inp, d, res = case(name)
    log(f"dispatch {name} cap={res.disp.cap}")
    idx = dev_tensor(res.routing.idx, "i32")
    got = moe.moe_dispatch(idx, cfg.E, cfg.capacity_factor)
    torch.cuda.synchronize()
    check_dispatch_equal({k: host_array(v) for k, v in got.items()}, res.disp)


@pytest.mark.parametrize("T,cf", [(1, None), (1000, None), (1000, 1.25), (3000, 0.3),
                                  (2048, 1.0), (1025, 1.25)])
def test_dispatch_concentrated_and_random(moe, T, cf):
    # half the tokens pick (0, 1) in either order, the rest random pairs:
    # exercises capacity drops, block boundaries (1024 tokens) and empty experts
    rng = np.random.default_rng(T)
    idx = np.empty((T, 2), np.int32)
    for t in range(T):
        if t % 2 == 0:
            idx[t] = (0, 1) if t % 4 == 0 else (1, 0)
        else:
            idx[t] = rng.choice(6, 2, replace=False) + 2
    ref = oracle.dispatch(idx, 8, cf)
    got = moe.moe_dispatch(dev_tensor(idx, "i32"), 8, cf)
    torch.cuda.synchronize()
    check_dispatch_equal({k: host_array(v) for k, v in got.items()}, ref)


@pytest.mark.parametrize("name", ALL)
def test_expert_ffn(moe, name):
    # the FFN on the oracle's dispatch: hidden rows and expert outputs
    cfg, inp, d, res = case(name)
    log(f"expert_ffn {name} T={cfg.T} H={cfg.H} F={cfg.F} {cfg.wdt}")
    perm = dev_tensor(res.disp.perm, "i32")
    off = dev_tensor(res.disp.offsets, "i32")
    h, y = moe.moe_expert_ffn(d["x"], perm, off, cfg.k, d["wg"], d["wu"], d["wd"],
                              d["sg"], d["su"], d["sd"])
    torch.cuda.synchronize()
    n = int(res.disp.offsets[-1])
    h_got, y_got = out_as_f64(h)[:n], out_as_f64(y)[:n]
    x64 = oracle.widen(inp.x, cfg.act)
    h_ref = np.zeros((n, cfg.F))
    y_ref = np.zeros((n, cfg.H))
    y_from_gpu_h = np.zeros((n, cfg.H))
    for e in range(cfg.E):
        r0, r1 = res.disp.offsets[e], res.disp.offsets[e + 1]
        if r1 == r0:
            continue
        tok = res.disp.perm[r0:r1] // cfg.k
        sc = (lambda a: None if a is None else a[e])
        wd64 = oracle.widen(inp.wd[e], cfg.wdt, sc(inp.sd))
        h_ref[r0:r1] = oracle.expert_hidden(x64[tok], oracle.widen(inp.wg[e], cfg.wdt, sc(inp.sg)),
                                            oracle.widen(inp.wu[e], cfg.wdt, sc(inp.su)))
        y_ref[r0:r1] = h_ref[r0:r1] @ wd64.T
        y_from_gpu_h[r0:r1] = h_got[r0:r1] @ wd64.T
    check_close(h_got, h_ref, cfg.act, "h")
    check_close(y_got, y_ref, cfg.act, "y_perm")
    # the down projection alone, from the GPU's own (rounded) h
    check_close(y_got, y_from_gpu_h, cfg.act, "y_perm from GPU h")


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_combine(moe, act):
    cfg, inp, d, res = case("p_cap")
    rng = np.random.default_rng(5)
    n = int(res.disp.offsets[-1])
    y32 = rng.standard_normal((cfg.T * cfg.k, cfg.H)).astype(np.float32)
    y_st = synth.bf16_bits_from_f32(y32) if act == "bf16" else y32
    y_dev = dev_tensor(y_st, act)
    w32 = res.routing.w.astype(np.float32)
    out = moe.moe_combine(y_dev, dev_tensor(res.disp.slot_row, "i32"), dev_tensor(w32, "f32"))
    torch.cuda.synchronize()
    y64 = oracle.widen(y_st, act)
    ref = oracle.combine(y64[:n], res.disp.slot_row, w32.astype(np.float64))
    check_close(out_as_f64(out), ref, act, "combine")
    dropped_rows = res.disp.dropped.reshape(cfg.T, cfg.k).all(axis=1)
    assert np.all(out_as_f64(out)[dropped_rows] == 0.0)


@pytest.mark.parametrize("name", ALL)
def test_layer_forward(moe, name):
    cfg, inp, d, res = case(name)
    log(f"layer {name} T={cfg.T} H={cfg.H} F={cfg.F} {cfg.act}/{cfg.wdt} cf={cfg.capacity_factor}")
    out, ax = moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=cfg.k,
                                    capacity_factor=cfg.capacity_factor, s_gate=d["sg"],
                                    s_up=d["su"], s_down=d["sd"], aux=True)
    torch.cuda.synchronize()
    w = host_array(ax["topk_w"])
    own = gpu_routing(host_array(ax["topk_idx"]), w, res.routing)
    if own is not None:
        res = oracle.layer_forward(inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt,
                                   k=cfg.k, capacity_factor=cfg.capacity_factor, sg=inp.sg,
                                   su=inp.su, sd=inp.sd, idx=own)
    check_weights(w, res.routing)
    # the layer's dispatch outputs, and the dispatch of the layer's own indices
    # (perm, slot_row), bit-exact against the oracle's dispatch of the same indices
    assert np.array_equal(host_array(ax["counts"]), res.disp.counts)
    assert np.array_equal(host_array(ax["offsets"]), res.disp.offsets)
    assert np.array_equal(host_array(ax["dropped"]), res.disp.dropped)
    got = moe.moe_dispatch(ax["topk_idx"], cfg.E, cfg.capacity_factor)
    torch.cuda.synchronize()
    check_dispatch_equal({k: host_array(v) for k, v in got.items()}, res.disp)
    check_close(out_as_f64(out), res.out, cfg.act, "out")
    if cfg.capacity_factor is not None:
        assert res.disp.dropped.sum() > 0


def test_layer_determinism(moe):
    cfg, inp, d, res = case("p_cap_i8")
    a = moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=2,
                              capacity_factor=cfg.capacity_factor, s_gate=d["sg"], s_up=d["su"],
                              s_down=d["sd"])
    b = moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=2,
                              capacity_factor=cfg.capacity_factor, s_gate=d["sg"], s_up=d["su"],
                              s_down=d["sd"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_layer_empty_input(moe):
    cfg, inp, d, res = case("p_bf16")
    x0 = d["x"][:0]
    out, ax = moe.moe_layer_forward(x0, d["wr"], d["wg"], d["wu"], d["wd"], aux=True)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.H)
    assert host_array(ax["counts"]).tolist() == [0] * 8
    assert host_array(ax["offsets"]).tolist() == [0] * 9


def test_layer_all_tokens_two_experts(moe):
    # router rows 0 and 1 dominate: every token goes to experts 0 and 1, so
    # those experts get T rows each (many tiles) and the other six none
    cfg = synth.get_config("p_bf16").with_(T=700)
    inp = synth.generate_host(cfg)
    # non-negative activations and large positive router rows 0 > 1
    inp.x = synth.bf16_bits_from_f32(np.abs(oracle.widen(inp.x, cfg.act)).astype(np.float32))
    inp.wr[0] = np.abs(inp.wr[0]) * 2 + 1.0
    inp.wr[1] = np.abs(inp.wr[1]) + 0.5
    res = oracle.layer_forward(inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt, k=2)
    assert res.disp.counts[0] == cfg.T and res.disp.counts[1] == cfg.T
    d = to_device(inp)
    for cf in (None, 1.0):
        ref = res if cf is None else oracle.layer_forward(
            inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt, k=2, capacity_factor=cf)
        out, ax = moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"],
                                        capacity_factor=cf, aux=True)
        torch.cuda.synchronize()
        assert np.array_equal(host_array(ax["offsets"]), ref.disp.offsets)
        assert np.array_equal(host_array(ax["dropped"]), ref.disp.dropped)
        check_close(out_as_f64(out), ref.out, cfg.act, f"out cf={cf}")
        if cf is not None:
            both = ref.disp.dropped.reshape(cfg.T, 2).all(axis=1)
            assert both.any() and np.all(out_as_f64(out)[both] == 0.0)
