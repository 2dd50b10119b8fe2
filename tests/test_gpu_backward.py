"""GPU parity of the training entry points (moe_layer_forward_train and
moe_layer_backward) against oracle.layer_backward.

At parity sizes every element of dx, dW_router, dW_gate, dW_up and dW_down
is compared with the float64 oracle (bf16 tolerance of the forward tests:
the GPU rounds dy, dh, [dg | du] and the per-row dx to bf16 on the way, each
a relative 2^-9, besides the bf16 outputs). At the Grok-1 training shape
(T = 8192, capacity 1.25) the oracle evaluates 256 sampled dx rows, 256
entries of each expert weight gradient and the whole router weight gradient
(which needs every kept slot's expert output, so every expert row runs
through the float64 oracle), and the dispatch kept in the reserve is compared
bit-exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.device import generate_device, grad_output_device
from gpu_helpers import (LazyExperts, check_close, check_weights, dev_tensor, gpu_routing,
                         host_array, log, out_as_f64, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_transformer_top_amd as m
    m.load_library()
    return m


def _run(moe, d, dout, cfg):
    out, res = moe.moe_layer_forward_train(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=cfg.k,
                                           capacity_factor=cfg.capacity_factor)
    g = moe.moe_layer_backward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], dout, res, k=cfg.k)
    torch.cuda.synchronize()
    return out, res, g


CASES = [
    synth.get_config("p_bf16"),
    synth.get_config("p_cap"),
    synth.get_config("p_bf16_tail"),
    synth.get_config("p_dec1"),
    synth.get_config("p_bf16_dec"),
    # k = 1 over 4 experts; k = 4 with a tight capacity (tokens lose all slots)
    synth.get_config("p_bf16").with_(name="k1", T=200, E=4, k=1, seed=31),
    synth.get_config("p_cap").with_(name="k4cap", T=190, k=4, capacity_factor=0.5, seed=32,
                                    skew=(3.0, 2.5)),
    # 40 column tiles in the dx-rows product and the forward down projection:
    # whole rounds plus tail tiles split along k on every XCD
    synth.get_config("p_bf16").with_(name="wide_tail", T=600, H=10240, F=256, seed=33),
]


def _random_cases(n=10, seed=77):
    """Seeded random training shapes: expert counts 1 … 16, k up to 4, sizes
    that are multiples of 64 but not of the 256-wide tiles, capacity factors
    that drop and that do not, skewed and plain routers."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        E = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
        k = int(rng.integers(1, min(E, 4) + 1))
        T = int(rng.integers(1, 17)) if c % 4 == 0 else int(rng.integers(17, 500))
        H = 64 * int(rng.integers(1, 11))
        F = 64 * int(rng.integers(1, 13))
        cf = [None, 0.5, 1.0, 1.25, 2.0][int(rng.integers(0, 5))]
        skew = (float(rng.uniform(1, 3)), float(rng.uniform(0.5, 2))) if rng.random() < 0.3 else ()
        cases.append(synth.LayerConfig(f"rb{c}_E{E}k{k}T{T}H{H}F{F}", T=T, H=H, F=F, E=E, k=k,
                                       capacity_factor=cf, skew=skew, seed=2000 + c))
    return cases


RANDOM_CASES = _random_cases()


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_backward_matches_oracle(moe, cfg):
    _check_backward(moe, cfg)


@pytest.mark.parametrize("cfg", RANDOM_CASES, ids=[c.name for c in RANDOM_CASES])
def test_backward_random_shapes(moe, cfg):
    _check_backward(moe, cfg)


def _check_backward(moe, cfg):
    log(f"backward {cfg.name}: T={cfg.T} H={cfg.H} F={cfg.F} E={cfg.E} k={cfg.k} "
        f"cf={cfg.capacity_factor}")
    inp = synth.generate_host(cfg)
    d = to_device(inp)
    dout_bits = synth.grad_output(cfg.T, cfg.H, seed=cfg.seed + 100)
    out, res, g = _run(moe, d, dev_tensor(dout_bits, "bf16"), cfg)
    ref = oracle.layer_backward(inp.x, "bf16", inp.wr, inp.wg, inp.wu, inp.wd, "bf16",
                                oracle.widen(dout_bits, "bf16"), k=cfg.k,
                                capacity_factor=cfg.capacity_factor)
    v = moe.train_reserve_views(res, cfg.T, cfg.H, cfg.F, cfg.E, cfg.k)
    assert np.array_equal(host_array(v["topk_idx"]), ref.routing.idx), "routing differs (tie)"
    assert np.array_equal(host_array(v["offsets"]), ref.disp.offsets)
    assert np.array_equal(host_array(v["slot_row"]), ref.disp.slot_row)
    check_close(out_as_f64(out), ref.out, "bf16", "out")
    for name, got, want in (("dx", g["dx"], ref.dx), ("dw_router", g["dw_router"], ref.dwr),
                            ("dw_gate", g["dw_gate"], ref.dwg), ("dw_up", g["dw_up"], ref.dwu),
                            ("dw_down", g["dw_down"], ref.dwd)):
        r = check_close(out_as_f64(got), want, "bf16", name)
        log(f"  {name}: max ratio {r[0]:.2e}, l2 ratio {r[1]:.2e}")
    # experts without rows have exactly zero weight gradients
    empty = np.diff(ref.disp.offsets) == 0
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert not out_as_f64(g[n])[empty].any()
    # a token whose slots were all dropped gets no gradient at all
    lost = ref.disp.dropped.reshape(cfg.T, cfg.k).all(axis=1)
    if lost.any():
        log(f"  tokens with every slot dropped: {int(lost.sum())}")
        assert not out_as_f64(g["dx"])[lost].any()


def test_train_forward_matches_layer_forward(moe):
    cfg = synth.get_config("p_cap")
    d = to_device(synth.generate_host(cfg))
    out, res = moe.moe_layer_forward_train(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=2,
                                           capacity_factor=cfg.capacity_factor)
    ref = moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=2,
                                capacity_factor=cfg.capacity_factor)
    torch.cuda.synchronize()
    # same tiled kernels (T > 16): bitwise equal; h and y_perm as moe_expert_ffn writes them
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    v = moe.train_reserve_views(res, cfg.T, cfg.H, cfg.F, cfg.E, 2)
    h, y = moe.moe_expert_ffn(d["x"], v["perm"], v["offsets"], 2, d["wg"], d["wu"], d["wd"])
    torch.cuda.synchronize()
    n = int(host_array(v["offsets"])[-1])
    assert torch.equal(h[:n].view(torch.int16), v["h"][:n].view(torch.int16))
    assert torch.equal(y[:n].view(torch.int16), v["y_perm"][:n].view(torch.int16))
    # h is silu(g) * u of the kept pre-activations, up to their bf16 rounding
    gg, uu = v["g"][:n].float(), v["u"][:n].float()
    hh = torch.nn.functional.silu(gg) * uu
    check_close(out_as_f64(hh), out_as_f64(h[:n]), "bf16", "h from g, u")


def test_backward_is_deterministic(moe):
    cfg = synth.get_config("p_skew")
    inp = synth.generate_host(cfg)
    d = to_device(inp)
    dout = dev_tensor(synth.grad_output(cfg.T, cfg.H, seed=5), "bf16")
    _, res, g1 = _run(moe, d, dout, cfg)
    g2 = moe.moe_layer_backward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], dout, res, k=2)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n].view(torch.int16) if g1[n].dtype == torch.bfloat16 else g1[n],
                           g2[n].view(torch.int16) if g2[n].dtype == torch.bfloat16 else g2[n]), n


def test_split_backward_equals_fused(moe):
    cfg = synth.get_config("p_cap")
    d = to_device(synth.generate_host(cfg))
    dout = dev_tensor(synth.grad_output(cfg.T, cfg.H, seed=6), "bf16")
    _, res, g1 = _run(moe, d, dout, cfg)
    g2 = moe.moe_layer_backward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], dout, res, k=2,
                                split=True)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n].view(torch.int16) if g1[n].dtype == torch.bfloat16 else g1[n],
                           g2[n].view(torch.int16) if g2[n].dtype == torch.bfloat16 else g2[n]), n


def test_backward_empty_batch(moe):
    cfg = synth.get_config("p_bf16").with_(T=0)
    d = to_device(synth.generate_host(cfg))
    dout = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    out, res, g = _run(moe, d, dout, cfg)
    assert out.shape == (0, cfg.H)
    for n in ("dw_router", "dw_gate", "dw_up", "dw_down"):
        assert not g[n].float().abs().sum().item(), n


# The Grok-1 training shape, and x above 2 GiB (4400 tokens of 245 760: the
# saving gate/up kernel's 64-bit row pointers, 2 GB of gathered rows in the
# backward) with a small F.
LARGE = [synth.CONFIGS["train"],
         synth.LayerConfig("train_wide_x", T=4400, H=245_760, F=128, capacity_factor=1.25,
                           seed=61)]


@pytest.mark.parametrize("cfg", LARGE, ids=[c.name for c in LARGE])
def test_backward_at_grok1_training_shape(moe, cfg):
    log(f"backward at {cfg.name}: T={cfg.T} H={cfg.H} F={cfg.F} cf={cfg.capacity_factor}")
    dv = generate_device(cfg, "cuda")
    d = dict(x=dv.x, wr=dv.wr, wg=dv.wg, wu=dv.wu, wd=dv.wd)
    dout = grad_output_device(cfg.T, cfg.H, seed=cfg.seed)
    out, res, g = _run(moe, d, dout, cfg)
    v = moe.train_reserve_views(res, cfg.T, cfg.H, cfg.F, cfg.E, cfg.k)
    x_h, wr_h = host_array(d["x"]), host_array(d["wr"])
    l32, l64 = oracle.router_logits(oracle.widen(x_h, "bf16"), wr_h)
    routing = oracle.top_k_softmax(l32, l64, cfg.k)
    # the reference follows the GPU's choice where a tie-flagged token was
    # ordered differently (both correct); every other token must agree
    own = gpu_routing(host_array(v["topk_idx"]), host_array(v["topk_w"]), routing)
    rng = np.random.default_rng(2)
    tokens = np.sort(rng.choice(cfg.T, min(256, cfg.T), replace=False))
    ent = {"dwg": [], "dwu": [], "dwd": []}
    for e in range(cfg.E):
        for _ in range(32):      # 256 entries per weight gradient
            ent["dwg"].append((e, int(rng.integers(cfg.F)), int(rng.integers(cfg.H))))
            ent["dwu"].append((e, int(rng.integers(cfg.F)), int(rng.integers(cfg.H))))
            ent["dwd"].append((e, int(rng.integers(cfg.H)), int(rng.integers(cfg.F))))
    log(f"  oracle: {len(tokens)} dx rows, 256 entries per weight gradient, the whole "
        "router gradient (every expert row evaluated)")
    ref = oracle.layer_backward_sampled(
        x_h, "bf16", wr_h, LazyExperts(d["wg"]), LazyExperts(d["wu"]), LazyExperts(d["wd"]),
        "bf16", oracle.widen(host_array(dout), "bf16"), k=cfg.k,
        capacity_factor=cfg.capacity_factor, tokens=tokens, entries=ent, idx=own,
        router_grad=True, progress=log)
    check_weights(host_array(v["topk_w"]), ref.routing)
    # the dispatch the forward kept in the reserve, bit-exact
    for n in ("counts", "offsets", "perm", "slot_row", "dropped"):
        assert np.array_equal(host_array(v[n]), getattr(ref.disp, n)), n
    log(f"  kept rows {int(ref.disp.offsets[-1])} of {cfg.T * cfg.k}")
    r = check_close(out_as_f64(g["dx"])[tokens], ref.dx, "bf16", "dx rows")
    log(f"  dx ({len(tokens)} rows): max ratio {r[0]:.2e}, l2 ratio {r[1]:.2e}")
    for n, key in (("dwg", "dw_gate"), ("dwu", "dw_up"), ("dwd", "dw_down")):
        ids, want = ref.entries[n]
        got = out_as_f64(g[key][ids[:, 0], ids[:, 1], ids[:, 2]])
        # each entry sums ~2000 rows whose factors were rounded to bf16 on the
        # way: the error scales with the entries' typical size, not with each
        # entry (the same bar as the dense comparisons, over the sample)
        r = check_close(got, want, "bf16", key)
        rel = np.abs(got - want) / np.maximum(np.abs(want), 1e-30)
        log(f"  {key} ({len(want)} entries): max ratio {r[0]:.2e}, l2 ratio {r[1]:.2e}; "
            f"per-entry relative error median {np.median(rel):.2e}, 99th pct "
            f"{np.quantile(rel, 0.99):.2e}")
    dwr = out_as_f64(g["dw_router"])
    r = check_close(dwr, ref.dwr, "bf16", "dw_router")
    log(f"  dw_router (all {dwr.size} entries): max ratio {r[0]:.2e}, l2 ratio {r[1]:.2e}")
    assert np.abs(dwr.sum(axis=0)).max() <= 1e-4 * np.abs(dwr).max()
    del dv, d, res, g
    torch.cuda.empty_cache()
