"""Pins of the oracle's layer backward (oracle.layer_backward), independent of
its own chain-rule derivation:

  * central finite differences of the oracle's forward (itself pinned in
    test_oracle_ffn / test_oracle_routing) for entries of every input and
    weight, on float32-stored inputs, with capacity drops and without;
  * torch autograd (float64, CPU) through a forward written here with torch
    ops, the routing decisions taken from the oracle;
  * closed forms: the layer is linear in W_down and in W_up, so
    sum(W * dW) equals the loss for each; the softmax Jacobian makes every
    token's logit gradient sum to zero, hence sum_e dWr[e] = 0; with one
    expert and k = 1 the routing weight is constantly 1, so dWr = 0 exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import LayerConfig


def _cfg(T, H, F, E, k, cf=None, act="f32", wdt="f32", seed=0):
    return LayerConfig("bwd", T=T, H=H, F=F, E=E, k=k, capacity_factor=cf, act=act,
                       wdt=wdt, seed=seed)


def _dout(cfg, seed=99):
    return np.random.default_rng(seed).standard_normal((cfg.T, cfg.H))


def _loss(inp, cfg, dout, **over):
    a = dict(x=inp.x, wr=inp.wr, wg=inp.wg, wu=inp.wu, wd=inp.wd)
    a.update(over)
    res = oracle.layer_forward(a["x"], cfg.act, a["wr"], a["wg"], a["wu"], a["wd"], cfg.wdt,
                               k=cfg.k, capacity_factor=cfg.capacity_factor)
    return float(np.sum(dout * res.out)), res


def _clear_margins(cfg, min_gap):
    """First seed whose float64 logit gaps (slot order and the k / k+1
    boundary) all exceed min_gap, so small perturbations keep the routing."""
    for seed in range(200):
        inp = synth.generate_host(cfg.with_(seed=seed))
        _, l64 = oracle.router_logits(oracle.widen(inp.x, cfg.act), inp.wr)
        r = -np.sort(-l64, axis=1)
        last = min(cfg.k, cfg.E - 1)
        if np.all(r[:, :last] - r[:, 1:last + 1] > min_gap):
            return inp
    raise AssertionError("no seed with clear routing margins")


def _perturbed(arr, index, eps):
    """(plus, minus, delta): float32 copies with arr[index] moved up / down by
    about eps, and the exact distance between the two stored values."""
    p, m = arr.copy(), arr.copy()
    p[index] = np.float32(float(arr[index]) + eps)
    m[index] = np.float32(float(arr[index]) - eps)
    return p, m, float(p[index]) - float(m[index])


@pytest.mark.parametrize("cf", [None, 0.75])
def test_backward_matches_finite_differences(cf):
    cfg = _cfg(T=9, H=8, F=12, E=4, k=2, cf=cf)
    inp = _clear_margins(cfg, 0.05)
    dout = _dout(cfg)
    L0, base = _loss(inp, cfg, dout)
    g = oracle.layer_backward(inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt, dout,
                              k=cfg.k, capacity_factor=cf)
    assert np.allclose(g.out, base.out, rtol=0, atol=1e-12)
    if cf is not None:
        assert g.disp.dropped.any()          # the case exercises the capacity drop
    rng = np.random.default_rng(1)
    eps = 2.0 ** -12
    grads = dict(x=g.dx, wr=g.dwr, wg=g.dwg, wu=g.dwu, wd=g.dwd)
    for name, grad in grads.items():
        arr = getattr(inp, name)
        flat = [np.unravel_index(i, arr.shape) for i in
                (range(arr.size) if arr.size <= 80 else rng.choice(arr.size, 80, replace=False))]
        for index in flat:
            p, m, delta = _perturbed(arr, index, eps)
            Lp, rp = _loss(inp, cfg, dout, **{name: p})
            Lm, rm = _loss(inp, cfg, dout, **{name: m})
            for r in (rp, rm):   # the routing must not move
                assert np.array_equal(r.routing.idx, base.routing.idx)
                assert np.array_equal(r.disp.slot_row, base.disp.slot_row)
            fd = (Lp - Lm) / delta
            assert abs(fd - grad[index]) <= 2e-6 * (1.0 + abs(grad[index])), (name, index)


def _torch_forward(x, wr, wg, wu, wd, idx, slot_row, k):
    """out[t] = sum over kept slots of softmax(selected logits)_j * expert(x_t)."""
    logits = x @ wr.T
    w = torch.softmax(torch.gather(logits, 1, idx), dim=1)
    T = x.shape[0]
    out = torch.zeros_like(x)
    for t in range(T):
        for j in range(k):
            if slot_row[t * k + j] < 0:
                continue
            e = int(idx[t, j])
            h = torch.nn.functional.silu(x[t] @ wg[e].T) * (x[t] @ wu[e].T)
            out = out.index_add(0, torch.tensor([t]), (w[t, j] * (h @ wd[e].T))[None])
    return out


@pytest.mark.parametrize("act,wdt,cf", [("f32", "f32", 1.0), ("bf16", "bf16", None)])
def test_backward_matches_torch_autograd(act, wdt, cf):
    cfg = _cfg(T=40, H=32, F=48, E=8, k=2, cf=cf, act=act, wdt=wdt, seed=5)
    inp = synth.generate_host(cfg)
    dout = _dout(cfg, seed=7)
    g = oracle.layer_backward(inp.x, act, inp.wr, inp.wg, inp.wu, inp.wd, wdt, dout,
                              k=cfg.k, capacity_factor=cf)
    if cf is not None:
        assert g.disp.dropped.any()
    leaf = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    x = leaf(oracle.widen(inp.x, act))
    wr = leaf(np.asarray(inp.wr, np.float64))
    wg = leaf(np.stack([oracle.widen(w, wdt) for w in inp.wg]))
    wu = leaf(np.stack([oracle.widen(w, wdt) for w in inp.wu]))
    wd = leaf(np.stack([oracle.widen(w, wdt) for w in inp.wd]))
    out = _torch_forward(x, wr, wg, wu, wd, torch.tensor(g.routing.idx, dtype=torch.int64),
                         g.disp.slot_row, cfg.k)
    (torch.tensor(dout) * out).sum().backward()
    for mine, ref in ((g.out, out.detach()), (g.dx, x.grad), (g.dwr, wr.grad),
                      (g.dwg, wg.grad), (g.dwu, wu.grad), (g.dwd, wd.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(mine - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("cf", [None, 1.25])
def test_backward_closed_forms(cf):
    cfg = _cfg(T=64, H=48, F=80, E=8, k=2, cf=cf, act="bf16", wdt="bf16", seed=11)
    inp = synth.generate_host(cfg)
    dout = _dout(cfg, seed=3)
    g = oracle.layer_backward(inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt, dout,
                              k=cfg.k, capacity_factor=cf)
    L = float(np.sum(dout * g.out))
    wd64 = np.stack([oracle.widen(w, "bf16") for w in inp.wd])
    wu64 = np.stack([oracle.widen(w, "bf16") for w in inp.wu])
    # out is linear in W_down and in W_up (h = silu(g) * u)
    assert abs(np.sum(wd64 * g.dwd) - L) <= 1e-11 * max(1.0, abs(L))
    assert abs(np.sum(wu64 * g.dwu) - L) <= 1e-11 * max(1.0, abs(L))
    # softmax over the selected logits: each token's logit gradient sums to 0
    assert np.max(np.abs(g.dlogits.sum(axis=1))) <= 1e-14 * max(1.0, np.abs(g.dlogits).max())
    assert np.max(np.abs(g.dwr.sum(axis=0))) <= 1e-12 * max(1.0, np.abs(g.dwr).max())
    # only selected logits get a gradient; dropped slots get none
    sel = np.zeros_like(g.dlogits, bool)
    np.put_along_axis(sel, g.routing.idx.astype(np.int64), True, axis=1)
    assert np.all(g.dlogits[~sel] == 0.0)
    dropped = g.disp.dropped.reshape(cfg.T, cfg.k).astype(bool)
    assert np.all(g.dw[dropped] == 0.0)


def test_backward_one_expert_has_no_router_gradient():
    cfg = _cfg(T=10, H=16, F=24, E=1, k=1, seed=2)
    inp = synth.generate_host(cfg)
    g = oracle.layer_backward(inp.x, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt,
                              _dout(cfg), k=1)
    assert np.all(g.routing.w == 1.0)
    assert np.all(g.dwr == 0.0) and np.all(g.dlogits == 0.0)
    # then dx is the plain SwiGLU MLP's input gradient: compare with autograd
    x = torch.tensor(oracle.widen(inp.x, "f32"), requires_grad=True)
    wg, wu, wd = (torch.tensor(np.asarray(a[0], np.float64)) for a in (inp.wg, inp.wu, inp.wd))
    y = (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)) @ wd.T
    (torch.tensor(_dout(cfg)) * y).sum().backward()
    assert np.max(np.abs(g.dx - x.grad.numpy())) <= 1e-12 * max(1.0, np.abs(g.dx).max())


def test_silu_grad_closed_form():
    g = np.array([-30.0, -2.5, -1e-3, 0.0, 1e-3, 0.7, 4.0, 30.0])
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5
    # central differences of silu itself
    h = 1e-5
    fd = (oracle.silu(g + h) - oracle.silu(g - h)) / (2 * h)
    assert np.allclose(oracle.silu_grad(g), fd, rtol=1e-8, atol=1e-10)


@pytest.mark.parametrize("cf", [None, 1.0])
def test_sampled_backward_equals_full(cf):
    # the per-entry evaluation used at sizes the full backward cannot reach
    cfg = _cfg(T=50, H=32, F=64, E=8, k=2, cf=cf, act="bf16", wdt="bf16", seed=21)
    inp = synth.generate_host(cfg)
    dout = synth.grad_output(cfg.T, cfg.H, seed=4)
    d64 = oracle.widen(dout, "bf16")
    g = oracle.layer_backward(inp.x, "bf16", inp.wr, inp.wg, inp.wu, inp.wd, "bf16", d64,
                              k=2, capacity_factor=cf)
    rng = np.random.default_rng(0)
    ent = {"dwg": [(int(rng.integers(8)), int(rng.integers(64)), int(rng.integers(32)))
                   for _ in range(20)],
           "dwu": [(int(rng.integers(8)), int(rng.integers(64)), int(rng.integers(32)))
                   for _ in range(20)],
           "dwd": [(int(rng.integers(8)), int(rng.integers(32)), int(rng.integers(64)))
                   for _ in range(20)]}
    tokens = np.array([0, 7, 19, 49])
    for router_grad in (False, True):
        s = oracle.layer_backward_sampled(inp.x, "bf16", inp.wr, inp.wg, inp.wu, inp.wd, "bf16",
                                          dout=d64, k=2, capacity_factor=cf, tokens=tokens,
                                          entries=ent, router_grad=router_grad)
        assert np.allclose(s.dx, g.dx[tokens], rtol=1e-12, atol=1e-12)
        for n, full in (("dwg", g.dwg), ("dwu", g.dwu), ("dwd", g.dwd)):
            ids, v = s.entries[n]
            assert np.allclose(v, full[ids[:, 0], ids[:, 1], ids[:, 2]], rtol=1e-12, atol=1e-13)
        if router_grad:
            # the whole router weight gradient, every token's logits
            assert np.max(np.abs(s.dwr - g.dwr)) <= 1e-12 * max(1.0, np.abs(g.dwr).max())
        else:
            assert s.dwr is None


def _other_choice(routing, E, seed):
    """Indices that differ from the top-k rule's for about a third of the
    tokens: slot 1 takes the third-ranked expert, or the two slots swap."""
    rng = np.random.default_rng(seed)
    idx = routing.idx.copy()
    order = np.argsort(-routing.l32, axis=1, kind="stable")
    for t in range(idx.shape[0]):
        r = rng.random()
        if r < 0.2:
            idx[t, 1] = order[t, 2]
        elif r < 0.35:
            idx[t] = idx[t, ::-1]
    return idx


@pytest.mark.parametrize("cf", [None, 0.75])
def test_given_indices_match_autograd(cf):
    # the layer on a routing that is not the top-k rule's (given indices):
    # torch autograd through the torch forward with the same selection, and
    # the sampled evaluation (whole router gradient) against the full one
    cfg = _cfg(T=36, H=24, F=40, E=6, k=2, cf=cf, act="bf16", wdt="bf16", seed=8)
    inp = synth.generate_host(cfg)
    dout = _dout(cfg, seed=12)
    l32, l64 = oracle.router_logits(oracle.widen(inp.x, "bf16"), inp.wr)
    idx = _other_choice(oracle.top_k_softmax(l32, l64, 2), cfg.E, seed=3)
    g = oracle.layer_backward(inp.x, "bf16", inp.wr, inp.wg, inp.wu, inp.wd, "bf16", dout,
                              k=2, capacity_factor=cf, idx=idx)
    assert np.array_equal(g.routing.idx, idx)
    if cf is not None:
        assert g.disp.dropped.any()
    leaf = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    x = leaf(oracle.widen(inp.x, "bf16"))
    wr = leaf(np.asarray(inp.wr, np.float64))
    wg = leaf(np.stack([oracle.widen(w, "bf16") for w in inp.wg]))
    wu = leaf(np.stack([oracle.widen(w, "bf16") for w in inp.wu]))
    wd = leaf(np.stack([oracle.widen(w, "bf16") for w in inp.wd]))
    slot_row = oracle.dispatch(idx, cfg.E, cf).slot_row
    out = _torch_forward(x, wr, wg, wu, wd, torch.tensor(idx, dtype=torch.int64), slot_row, 2)
    (torch.tensor(dout) * out).sum().backward()
    for mine, ref in ((g.out, out.detach()), (g.dx, x.grad), (g.dwr, wr.grad),
                      (g.dwg, wg.grad), (g.dwu, wu.grad), (g.dwd, wd.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(mine - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())
    s = oracle.layer_backward_sampled(inp.x, "bf16", inp.wr, inp.wg, inp.wu, inp.wd, "bf16",
                                      dout=dout, k=2, capacity_factor=cf,
                                      tokens=np.array([1, 20, 35]), entries={}, idx=idx,
                                      router_grad=True)
    assert np.max(np.abs(s.dwr - g.dwr)) <= 1e-12 * max(1.0, np.abs(g.dwr).max())
    assert np.allclose(s.dx, g.dx[[1, 20, 35]], rtol=1e-12, atol=1e-12)
