"""Pins of the oracle's expert FFN and weighted combine (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _layer(inp, cfg, **kw):
    return oracle.layer_forward(inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt,
                                k=cfg.k, capacity_factor=cfg.capacity_factor,
                                sg=inp.sg, su=inp.su, sd=inp.sd, **kw)


def _dense_masked_reference(inp, cfg, res):
    """Every expert on every token (torch fp64 Linear/SiLU), then
    out = sum_e G[t,e] f_e(x_t) with G the kept routing weights."""
    x = torch.from_numpy(oracle.widen(inp.x, cfg.act))
    T = x.shape[0]
    G = np.zeros((T, cfg.E))
    for t in range(T):
        for j in range(cfg.k):
            if not res.disp.dropped[t * cfg.k + j]:
                G[t, res.routing.idx[t, j]] += res.routing.w[t, j]
    out = torch.zeros_like(x)
    for e in range(cfg.E):
        s = (lambda a: None if a is None else a[e])
        wg = torch.from_numpy(oracle.widen(inp.wg[e], cfg.wdt, s(inp.sg)))
        wu = torch.from_numpy(oracle.widen(inp.wu[e], cfg.wdt, s(inp.su)))
        wd = torch.from_numpy(oracle.widen(inp.wd[e], cfg.wdt, s(inp.sd)))
        f = torch.nn.functional.linear(
            torch.nn.functional.silu(torch.nn.functional.linear(x, wg)) *
            torch.nn.functional.linear(x, wu), wd)
        out += torch.from_numpy(G[:, e])[:, None] * f
    return out.numpy()


@pytest.mark.parametrize("name", ["tiny", "p_cap", "p_i8", "p_cap_i8", "p_i4_dec"])
def test_dense_masked_brute_force(name):
    cfg = synth.get_config(name)
    if cfg.T * cfg.H * cfg.F > 80_000_000:
        cfg = cfg.with_(T=64)
    inp = synth.generate_host(cfg)
    res = _layer(inp, cfg)
    ref = _dense_masked_reference(inp, cfg, res)
    assert np.max(np.abs(res.out - ref)) <= 1e-10 * max(1.0, np.abs(ref).max())
    if cfg.capacity_factor is not None:
        assert res.disp.dropped.sum() > 0


def test_given_indices_dense_masked_brute_force():
    # a routing that is not the top-k rule's: the dense-masked reference with
    # weights from torch's softmax over the same selected logits
    cfg = synth.get_config("p_cap").with_(T=96, capacity_factor=0.75)
    inp = synth.generate_host(cfg)
    x64 = oracle.widen(inp.x, cfg.act)
    l32, l64 = oracle.router_logits(x64, inp.wr)
    rng = np.random.default_rng(4)
    idx = np.stack([rng.choice(cfg.E, 2, replace=False) for _ in range(cfg.T)]).astype(np.int32)
    res = _layer(inp, cfg, idx=idx)
    assert np.array_equal(res.routing.idx, idx) and res.disp.dropped.any()
    w = torch.softmax(torch.gather(torch.from_numpy(l64), 1, torch.from_numpy(idx).long()),
                      dim=1).numpy()
    assert np.allclose(res.routing.w, w, rtol=0, atol=1e-15)
    ref = _dense_masked_reference(inp, cfg, res)
    assert np.max(np.abs(res.out - ref)) <= 1e-10 * max(1.0, np.abs(ref).max())
    # the top-k rule's own indices reproduce the default routing exactly
    own = _layer(inp, cfg)
    again = _layer(inp, cfg, idx=own.routing.idx)
    assert np.array_equal(again.routing.w, own.routing.w) and np.array_equal(again.out, own.out)
    with pytest.raises(ValueError):
        _layer(inp, cfg, idx=np.zeros((cfg.T, 2), np.int32))     # one expert twice


def test_sampled_tokens_equal_full_rows():
    cfg = synth.get_config("p_cap")
    inp = synth.generate_host(cfg)
    full = _layer(inp, cfg)
    sample = np.sort(np.random.default_rng(1).choice(cfg.T, 40, replace=False))
    part = _layer(inp, cfg, tokens=sample)
    assert np.array_equal(part.out, full.out[sample])


def test_identical_experts_closed_form():
    # all experts share one weight set: out = f(x) because kept weights sum to 1
    cfg = synth.get_config("tiny")
    inp = synth.generate_host(cfg)
    for a in (inp.wg, inp.wu, inp.wd):
        a[:] = a[0]
    res = _layer(inp, cfg)
    x = oracle.widen(inp.x, cfg.act)
    g = x @ inp.wg[0].astype(np.float64).T
    u = x @ inp.wu[0].astype(np.float64).T
    f = (g * (1.0 / (1.0 + np.exp(-g))) * u) @ inp.wd[0].astype(np.float64).T
    assert np.max(np.abs(res.out - f)) <= 1e-12 * np.abs(f).max()


def test_scalar_h1_f1_case():
    # H = F = 1: out = sum_j w_j * c_e * silu(a_e x) * (b_e x)
    E, k, T = 8, 2, 9
    rng = np.random.default_rng(7)
    x = rng.standard_normal((T, 1)).astype(np.float32)
    wr = rng.standard_normal((E, 1)).astype(np.float32)
    a = rng.standard_normal((E, 1, 1)).astype(np.float32)
    b = rng.standard_normal((E, 1, 1)).astype(np.float32)
    c = rng.standard_normal((E, 1, 1)).astype(np.float32)
    res = oracle.layer_forward(x, "f32", wr, a, b, c, "f32", k=k)
    for t in range(T):
        xv = float(x[t, 0])
        l = [xv * float(wr[e, 0]) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-l[e], e))[:k]
        z = [math.exp(l[e] - l[order[0]]) for e in order]
        ref = 0.0
        for j, e in enumerate(order):
            g = float(a[e, 0, 0]) * xv
            ref += z[j] / sum(z) * float(c[e, 0, 0]) * (g / (1 + math.exp(-g))) * float(b[e, 0, 0]) * xv
        assert abs(res.out[t, 0] - ref) <= 1e-13 * max(1.0, abs(ref))


def test_linearity_in_w_down():
    cfg = synth.get_config("tiny")
    inp = synth.generate_host(cfg)
    r1 = _layer(inp, cfg)
    inp.wd *= 2.0
    r2 = _layer(inp, cfg)
    assert np.array_equal(r2.out, 2.0 * r1.out)


def test_zero_up_removes_expert():
    cfg = synth.get_config("tiny")
    inp = synth.generate_host(cfg)
    base = _layer(inp, cfg)
    e0 = 3
    inp.wu[e0] = 0.0
    res = _layer(inp, cfg)
    ref = _dense_masked_reference(inp, cfg, res)
    assert np.max(np.abs(res.out - ref)) < 1e-12
    hit = np.any(base.routing.idx == e0, axis=1)
    assert hit.any()
    assert not np.allclose(res.out[hit], base.out[hit])
    assert np.array_equal(res.out[~hit], base.out[~hit])


def test_all_slots_dropped_gives_zero_row():
    # skewed capacity case: find tokens with both slots dropped
    cfg = synth.get_config("p_cap").with_(capacity_factor=0.4)
    inp = synth.generate_host(cfg)
    res = _layer(inp, cfg)
    both = res.disp.dropped.reshape(cfg.T, cfg.k).all(axis=1)
    assert both.any()
    assert np.all(res.out[both] == 0.0)
    assert np.all(np.abs(res.out[~both]).max(axis=1) > 0)


def test_silu_values():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert oracle.silu(np.array([800.0]))[0] == 800.0
    v = oracle.silu(np.array([-800.0]))[0]
    assert v == 0.0
    t = torch.linspace(-20, 20, 401, dtype=torch.float64)
    assert torch.allclose(torch.from_numpy(oracle.silu(t.numpy())),
                          torch.nn.functional.silu(t), rtol=1e-15, atol=1e-300)


def test_widen_int8_and_bf16():
    q = np.array([[-127, 0, 5], [127, -1, 2]], np.int8)
    s = np.array([0.5, 0.25], np.float32)
    assert oracle.widen(q, "i8", s).tolist() == [[-63.5, 0.0, 2.5], [31.75, -0.25, 0.5]]
    # bf16 bit patterns: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3F81 = 1 + 2^-7
    b = np.array([0x3F80, 0xC000, 0x3F81], np.uint16)
    assert oracle.widen(b, "bf16").tolist() == [1.0, -2.0, 1.0 + 2.0 ** -7]
    # matches torch's bfloat16 -> float64 conversion
    t = torch.randn(1000).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.widen(bits, "bf16"), t.to(torch.float64).numpy())


def test_widen_int4_hand_packed():
    # one row of K = 256 (two scale groups). Byte j holds k = 2j (low nibble)
    # and k = 2j+1 (high nibble); a nibble u means u - 8.
    packed = np.full((1, 128), 0x88, np.uint8)          # every code 8: value 0
    packed[0, 0] = 0x8F        # k0 = 15-8 = 7,  k1 = 8-8 = 0
    packed[0, 1] = 0x18        # k2 = 8-8 = 0,   k3 = 1-8 = -7
    packed[0, 63] = 0xF1       # k126 = -7,      k127 = 7
    packed[0, 64] = 0x9C       # k128 = 12-8 = 4, k129 = 9-8 = 1 (second group)
    packed[0, 127] = 0x08      # k254 = 0,       k255 = -8 (code 0)
    s = np.array([[0.5, 3.0]], np.float32)
    w = oracle.widen(packed, "i4", s)
    assert w.shape == (1, 256)
    want = np.zeros(256)
    want[[0, 3, 126, 127, 128, 129, 255]] = [3.5, -3.5, -3.5, 3.5, 12.0, 3.0, -24.0]
    assert np.array_equal(w[0], want)


def test_int4_quantisation_round_trip():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((5, 384)) * rng.uniform(0.01, 3.0, (5, 1))).astype(np.float32)
    w[2, 128:256] = 0.0                                  # an all-zero group
    packed, s = synth.quantize_int4_groups(w)
    assert packed.shape == (5, 192) and s.shape == (5, 3)
    back = oracle.widen(packed, "i4", s)
    g = w.reshape(5, 3, 128).astype(np.float64)
    err = np.abs(back.reshape(5, 3, 128) - g)
    # rounding to the nearest multiple of s: at most s/2 (plus float32 rounding of w/s)
    assert np.all(err <= (s.astype(np.float64) * (0.5 + 1e-6))[:, :, None])
    # the group's largest |w| maps to +-7 s
    amax = np.abs(g).argmax(axis=2)
    top = np.take_along_axis(back.reshape(5, 3, 128), amax[:, :, None], axis=2)[:, :, 0]
    assert np.array_equal(np.abs(top), 7.0 * s.astype(np.float64))
    assert np.all(back[2, 128:256] == 0.0) and s[2, 1] == 0.0
    # codes stay in 1 ... 15 (values -7 ... 7)
    codes = np.concatenate([packed & 15, packed >> 4])
    assert codes.min() >= 1 and codes.max() <= 15


def test_combine_and_hidden_agree_with_layer():
    # expert_hidden @ Wd^T per dispatched row, then combine == layer_forward
    cfg = synth.get_config("p_cap")
    inp = synth.generate_host(cfg)
    res = _layer(inp, cfg)
    x = oracle.widen(inp.x, cfg.act)
    n_rows = int(res.disp.offsets[-1])
    y = np.zeros((cfg.T * cfg.k, cfg.H))
    for e in range(cfg.E):
        rows = np.arange(res.disp.offsets[e], res.disp.offsets[e + 1])
        if rows.size == 0:
            continue
        tok = res.disp.perm[rows] // cfg.k
        h = oracle.expert_hidden(x[tok], oracle.widen(inp.wg[e], cfg.wdt),
                                 oracle.widen(inp.wu[e], cfg.wdt))
        y[rows] = h @ oracle.widen(inp.wd[e], cfg.wdt).T
    out = oracle.combine(y[:n_rows], res.disp.slot_row, res.routing.w)
    assert np.max(np.abs(out - res.out)) < 1e-12 * np.abs(res.out).max()


def test_combine_hand_case():
    # two tokens, k = 2: token 0 keeps rows 1 and 0; token 1 drops slot 1
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    slot_row = np.array([1, 0, 2, -1])
    w = np.array([[0.75, 0.25], [0.6, 0.4]])
    out = oracle.combine(y, slot_row, w)
    assert out.tolist() == [[7.75, 15.5], [60.0, 120.0]]
