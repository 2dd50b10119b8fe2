"""GPU parity for shapes beyond the Grok-1 defaults and for the ABI's stage
entry points: other expert counts and k, the decode/tiled kernel boundary
(T = 16 / 17), empty experts, experts with few rows on either tile shape, and
moe_expert_gate_up / moe_expert_down called on their own."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (check_close, check_dispatch_equal, check_routing, dev_tensor,
                         gpu_routing, host_array, log, out_as_f64, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_transformer_top_amd as m
    m.load_library()
    return m


def run_layer(moe, cfg, inp, d):
    out, ax = moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=cfg.k,
                                    capacity_factor=cfg.capacity_factor, s_gate=d["sg"],
                                    s_up=d["su"], s_down=d["sd"], aux=True)
    torch.cuda.synchronize()
    res = oracle.layer_forward(inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt, k=cfg.k,
                               capacity_factor=cfg.capacity_factor, sg=inp.sg, su=inp.su,
                               sd=inp.sd)
    return out, ax, res


SHAPES = [
    # name, T, H, F, E, k, act, wdt, cf
    ("e16_k4", 200, 256, 384, 16, 4, "bf16", "bf16", None),
    ("e16_k4_dec", 12, 256, 384, 16, 4, "bf16", "bf16", None),
    ("e4_k1", 150, 192, 320, 4, 1, "bf16", "bf16", None),
    ("e4_k1_cap", 150, 192, 320, 4, 1, "bf16", "i8", 1.1),
    ("e12_k3_f32", 70, 128, 256, 12, 3, "f32", "f32", 2.0),
    ("t16_dec", 16, 512, 640, 8, 2, "bf16", "bf16", None),
    ("t17_tiled", 17, 512, 640, 8, 2, "bf16", "bf16", None),
    ("t16_dec_i8", 16, 512, 640, 8, 2, "bf16", "i8", None),
    ("e2_k2", 90, 256, 256, 2, 2, "bf16", "bf16", 0.75),
    # T <= 8, bf16: the gate/up kernel with the token rows in LDS; ragged F
    # (idle waves in the last work-group), H not a multiple of 128, E = 16
    ("t8_lds_tail", 8, 320, 448, 8, 2, "bf16", "bf16", None),
    ("t3_lds_e16k4", 3, 256, 384, 16, 4, "bf16", "bf16", None),
    # rows too wide for LDS: falls back to the split-k decode kernel
    ("t8_wide_h", 8, 10240, 128, 8, 2, "bf16", "bf16", None),
    ("t8_i8_i4", 8, 384, 256, 8, 2, "bf16", "i4", None),
    # 40 column tiles of the down projection per row tile: each XCD runs one
    # whole round of 32 tiles and splits its 8 tail tiles along k (4 pieces)
    ("t600_tail_split", 600, 10240, 256, 8, 2, "bf16", "bf16", None),
    # decode weight streams: int8 rows that are not a multiple of 128 bytes
    # (64-byte steps) next to full-line double steps, int4 with an odd number
    # of scale groups in one matrix and an even number in the other
    ("t5_i8_h320", 5, 320, 448, 8, 2, "bf16", "i8", None),
    ("t9_i8_f576", 9, 512, 576, 8, 2, "bf16", "i8", None),
    # int4 double steps over long rows: gate/up at H = 8448 (66 scale groups
    # per row), down at F = 65792 (514 groups, 257 double steps over 8 k
    # splits: a ragged last split)
    ("t4_i4_h8448", 4, 8448, 256, 8, 2, "bf16", "i4", None),
    ("t4_i4_f65792", 4, 256, 65792, 8, 2, "bf16", "i4", None),
    # int4 gate/up scales staged in LDS in 256-byte pieces per 16-row tile:
    # H = 768 gives 6 groups per row, 96 scales per tile, a full and a
    # partial piece (H = 256 above: one partial piece and three waves without
    # a double step; H = 8448: 66 groups, past the table, read from memory)
    ("t6_i4_h768", 6, 768, 384, 8, 2, "bf16", "i4", None),
    ("t8_i4_mixed", 8, 512, 640, 8, 2, "bf16", "i4", None),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_layer_shapes(moe, shape):
    name, T, H, F, E, k, act, wdt, cf = shape
    cfg = synth.LayerConfig(name, T=T, H=H, F=F, E=E, k=k, act=act, wdt=wdt,
                            capacity_factor=cf, seed=len(name))
    log(f"shape {name}")
    inp = synth.generate_host(cfg)
    out, ax, res = run_layer(moe, cfg, inp, to_device(inp))
    diff = check_routing(host_array(ax["topk_idx"]), host_array(ax["topk_w"]), res.routing)
    assert not diff.any()
    assert np.array_equal(host_array(ax["counts"]), res.disp.counts)
    assert np.array_equal(host_array(ax["offsets"]), res.disp.offsets)
    assert np.array_equal(host_array(ax["dropped"]), res.disp.dropped)
    check_close(out_as_f64(out), res.out, act, name)


def test_dispatch_on_oracle_indices_general_k(moe):
    rng = np.random.default_rng(3)
    # 1024 tokens fill exactly one dispatch block (single-kernel path); 1025 need two
    for T, E, k, cf in ((3000, 16, 4, 1.0), (2500, 4, 1, 1.5), (777, 12, 3, None),
                        (1024, 8, 2, 1.25), (1025, 8, 2, 1.25), (1, 8, 2, 1.25)):
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        got = moe.moe_dispatch(dev_tensor(idx, "i32"), E, cf)
        torch.cuda.synchronize()
        check_dispatch_equal({n: host_array(v) for n, v in got.items()}, oracle.dispatch(idx, E, cf))


@pytest.mark.parametrize("name", ["p_bf16", "p_i8", "p_bf16_dec", "p_i8_dec", "p_i4_dec"])
def test_stage_entry_points(moe, name):
    # moe_expert_gate_up then moe_expert_down, each against the oracle
    cfg = synth.get_config(name)
    inp = synth.generate_host(cfg)
    d = to_device(inp)
    res = oracle.layer_forward(inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt, k=cfg.k,
                               sg=inp.sg, su=inp.su, sd=inp.sd)
    perm = dev_tensor(res.disp.perm, "i32")
    off = dev_tensor(res.disp.offsets, "i32")
    h = moe.moe_expert_gate_up(d["x"], perm, off, cfg.k, d["wg"], d["wu"], d["sg"], d["su"])
    y = moe.moe_expert_down(h, off, cfg.T, cfg.k, d["wd"], d["sd"])
    torch.cuda.synchronize()
    n = int(res.disp.offsets[-1])
    x64 = oracle.widen(inp.x, cfg.act)
    hg, yg = out_as_f64(h)[:n], out_as_f64(y)[:n]
    h_ref = np.zeros_like(hg)
    y_ref = np.zeros_like(yg)
    for e in range(cfg.E):
        r0, r1 = res.disp.offsets[e], res.disp.offsets[e + 1]
        if r1 == r0:
            continue
        sc = (lambda a: None if a is None else a[e])
        tok = res.disp.perm[r0:r1] // cfg.k
        h_ref[r0:r1] = oracle.expert_hidden(x64[tok], oracle.widen(inp.wg[e], cfg.wdt, sc(inp.sg)),
                                            oracle.widen(inp.wu[e], cfg.wdt, sc(inp.su)))
        y_ref[r0:r1] = hg[r0:r1] @ oracle.widen(inp.wd[e], cfg.wdt, sc(inp.sd)).T
    check_close(hg, h_ref, cfg.act, "gate_up")
    check_close(yg, y_ref, cfg.act, "down")


@pytest.mark.parametrize("name", ["p_bf16", "p_bf16_dec", "p_i8", "p_i4_dec"])
def test_determinism_each_path(moe, name):
    cfg = synth.get_config(name)
    d = to_device(synth.generate_host(cfg))
    outs = [moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=cfg.k,
                                  s_gate=d["sg"], s_up=d["su"], s_down=d["sd"]) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_router_logits_output(moe):
    cfg = synth.get_config("p_skew")
    inp = synth.generate_host(cfg)
    d = to_device(inp)
    idx, w, logits = moe.moe_router_topk(d["x"], d["wr"], 2, return_logits=True)
    torch.cuda.synchronize()
    l32, l64 = oracle.router_logits(oracle.widen(inp.x, cfg.act), inp.wr)
    lg = host_array(logits).astype(np.float64)
    assert np.max(np.abs(lg - l64) / np.maximum(1.0, np.abs(l64).max(axis=1, keepdims=True))) < 2e-5


def test_gather_over_2gib_of_x(moe):
    # x above 2 GiB: the gate/up kernel addresses the gathered rows with
    # 64-bit pointers instead of 32-bit offsets from x
    from synth.device import generate_device
    cfg = synth.LayerConfig("x_2gib", T=180_000, H=6144, F=128, E=8, k=2, seed=11)
    assert cfg.T * cfg.H * 2 > 2 ** 31
    log(f"x over 2 GiB: T={cfg.T} H={cfg.H} F={cfg.F}")
    d = generate_device(cfg, "cuda")
    out, ax = moe.moe_layer_forward(d.x, d.wr, d.wg, d.wu, d.wd, k=cfg.k, aux=True)
    torch.cuda.synchronize()
    sample = np.sort(np.random.default_rng(2).choice(cfg.T, 256, replace=False))
    # the oracle gets every token's routing; its FFN runs on the sample
    sample = np.concatenate([sample, [cfg.T - 1]]) if sample[-1] != cfg.T - 1 else sample
    res = oracle.layer_forward(host_array(d.x), cfg.act, host_array(d.wr), host_array(d.wg),
                               host_array(d.wu), host_array(d.wd), cfg.wdt, k=cfg.k,
                               tokens=sample)
    diff = check_routing(host_array(ax["topk_idx"]), host_array(ax["topk_w"]), res.routing)
    keep = ~diff[sample]
    if not diff.any():
        assert np.array_equal(host_array(ax["counts"]), res.disp.counts)
        assert np.array_equal(host_array(ax["offsets"]), res.disp.offsets)
    check_close(out_as_f64(out)[sample][keep], res.out[keep], cfg.act, "x over 2 GiB")
    del d, out, ax
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["p_bf16_dec", "p_dec1", "p_i8_dec", "p_i4_dec", "p_i4_dec16"])
def test_layer_forward_equals_stage_calls(moe, name):
    # The layer forward equals, bitwise, its stage entry points run one after
    # the other (router, dispatch, gate/up, down with its split-k reduce to
    # y_perm, combine) on the decode kernels with every weight type.
    cfg = synth.get_config(name)
    log(f"layer vs stage calls {name}: T={cfg.T} {cfg.wdt} cf={cfg.capacity_factor}")
    d = to_device(synth.generate_host(cfg))
    out = moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=cfg.k,
                                capacity_factor=cfg.capacity_factor, s_gate=d["sg"],
                                s_up=d["su"], s_down=d["sd"])
    idx, w = moe.moe_router_topk(d["x"], d["wr"], cfg.k)
    disp = moe.moe_dispatch(idx, cfg.E, cfg.capacity_factor)
    h = moe.moe_expert_gate_up(d["x"], disp["perm"], disp["offsets"], cfg.k, d["wg"], d["wu"],
                               d["sg"], d["su"])
    y = moe.moe_expert_down(h, disp["offsets"], cfg.T, cfg.k, d["wd"], d["sd"])
    ref = moe.moe_combine(y, disp["slot_row"], w)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("cf", [None, 1.0])
def test_few_row_experts_above_the_stream_threshold(moe, cf):
    # 2100 tokens over 8 experts: a mean of 525 rows per expert, above the
    # 256 up to which experts with at most 128 rows take the stream tiles, so
    # every expert runs on the wide tiles. The router makes three experts
    # small (32, 60 and 40 rows: tiles that fit their first half) next to
    # experts of 293 to 1212 rows; with cf = 1.0 the large ones drop rows.
    cfg = synth.get_config("p_bf16").with_(name="few_rows", T=2100, H=256, F=512, seed=93,
                                           capacity_factor=cf)
    inp = synth.generate_host(cfg)
    x = np.abs(oracle.widen(inp.x, "bf16")).astype(np.float32)
    x[:, :2] = 0.0
    x[:60, 0] = 1.0          # tokens 0..59 choose expert 6 first
    x[60:100, 1] = 1.0       # tokens 60..99 choose expert 7 first
    inp.x = synth.bf16_bits_from_f32(x)
    for e, f in ((6, 0), (7, 1)):
        inp.wr[e] = -np.abs(inp.wr[e])
        inp.wr[e][f] = 50.0
    d = to_device(inp)
    out, ax = moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=2,
                                    capacity_factor=cf, aux=True)
    torch.cuda.synchronize()
    res = oracle.layer_forward(inp.x, "bf16", inp.wr, inp.wg, inp.wu, inp.wd, "bf16", k=2,
                               capacity_factor=cf)
    own = gpu_routing(host_array(ax["topk_idx"]), host_array(ax["topk_w"]), res.routing)
    if own is not None:
        res = oracle.layer_forward(inp.x, "bf16", inp.wr, inp.wg, inp.wu, inp.wd, "bf16", k=2,
                                   capacity_factor=cf, idx=own)
    rows = np.diff(res.disp.offsets)
    log(f"few-row experts, cf={cf}: rows per expert {rows.tolist()}")
    assert cfg.T * 2 > 8 * 256 and (rows <= 128).sum() >= 3 and (rows > 256).sum() >= 3
    assert np.array_equal(host_array(ax["offsets"]), res.disp.offsets)
    assert np.array_equal(host_array(ax["dropped"]), res.disp.dropped)
    got = moe.moe_dispatch(ax["topk_idx"], 8, cf)
    torch.cuda.synchronize()
    check_dispatch_equal({k: host_array(v) for k, v in got.items()}, res.disp)
    check_close(out_as_f64(out), res.out, "bf16", f"few-row experts cf={cf}")
