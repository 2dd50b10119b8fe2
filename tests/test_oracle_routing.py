"""Pins of the oracle's router, top-k and softmax (CPU only).

Each check fixes the oracle against something other than itself: brute force
over all expert subsets, closed forms, library softmax, and hand-derived values.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
import synth


def _random_logits(T, E, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    l64 = rng.standard_normal((T, E)) * scale
    return l64.astype(np.float32), l64.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_topk_set_matches_brute_force_subsets(k):
    # The top-k set maximises the sum of its logits over all C(E,k) subsets.
    l32, l64 = _random_logits(400, 8, seed=11)
    r = oracle.top_k_softmax(l32, l64, k)
    for t in range(400):
        if r.tie[t]:
            continue
        best = max(itertools.combinations(range(8), k), key=lambda s: sum(l64[t, list(s)]))
        assert set(r.idx[t].tolist()) == set(best)


def test_slot_order_descending_and_distinct():
    l32, l64 = _random_logits(500, 8, seed=12)
    r = oracle.top_k_softmax(l32, l64, 2)
    assert np.all(r.idx[:, 0] != r.idx[:, 1])
    a = np.take_along_axis(l32, r.idx.astype(np.int64), axis=1)
    assert np.all(a[:, 0] >= a[:, 1])
    # slot 0 is the arg-max of the row
    assert np.array_equal(r.idx[:, 0], np.argmax(l32, axis=1))


def test_weights_sum_to_one_and_bounds():
    l32, l64 = _random_logits(1000, 8, seed=13, scale=3.0)
    r = oracle.top_k_softmax(l32, l64, 2)
    s = r.w.sum(axis=1)
    assert np.max(np.abs(s - 1.0)) <= 4 * np.finfo(np.float64).eps
    assert np.all(r.w[:, 0] >= 0.5) and np.all(r.w[:, 0] <= 1.0)
    assert np.all(r.w[:, 0] >= r.w[:, 1])


def test_weights_equal_renormalised_full_softmax():
    # softmax over the selected logits == full E-way softmax renormalised
    # over the selected experts (the common factor cancels)
    l32, l64 = _random_logits(300, 8, seed=14, scale=2.0)
    r = oracle.top_k_softmax(l32, l64, 2)
    p = sp_softmax(l64, axis=1)
    sel = np.take_along_axis(p, r.idx.astype(np.int64), axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    assert np.max(np.abs(ref - r.w)) < 1e-14


def test_zero_router_all_ties_lower_index_wins():
    # Wr = 0: every logit is 0, so experts 0 and 1 win with weights 1/2 each
    x = np.random.default_rng(0).standard_normal((17, 64)).astype(np.float32)
    wr = np.zeros((8, 64), np.float32)
    l32, l64 = oracle.router_logits(x.astype(np.float64), wr)
    r = oracle.top_k_softmax(l32, l64, 2)
    assert np.all(r.idx == np.array([0, 1]))
    assert np.all(r.w == 0.5)
    assert np.all(r.tie)


def test_hand_derived_ln3_case():
    # logits (0, ln 3, 0, 0, 0, 0, 0, -1): top-1 = expert 1; the remaining
    # zeros tie and the lowest index (0) wins; softmax(ln 3, 0) = (3/4, 1/4)
    l64 = np.array([[0.0, math.log(3.0), 0, 0, 0, 0, 0, -1.0]])
    l32 = l64.astype(np.float32)
    r = oracle.top_k_softmax(l32, l32.astype(np.float64), 2)
    assert r.idx.tolist() == [[1, 0]]
    assert abs(r.w[0, 0] - 0.75) < 1e-7 and abs(r.w[0, 1] - 0.25) < 1e-7
    assert r.tie[0]   # the 2nd / 3rd gap is 0


def test_tie_flags():
    l64 = np.array([[2.0, 1.0, 1.0 - 5e-5, -1, -1, -1, -1, -1],   # 2nd/3rd gap tiny
                    [2.0, 2.0 - 5e-5, 0.0, -1, -1, -1, -1, -1],   # 1st/2nd gap tiny
                    [2.0, 1.0, 0.0, -1, -1, -1, -1, -1]])         # clear
    r = oracle.top_k_softmax(l64.astype(np.float32), l64, 2)
    assert r.tie.tolist() == [True, True, False]


def test_router_logits_closed_form():
    # one-hot token rows pick out router columns; a row of ones sums them
    H, E = 32, 8
    wr = np.random.default_rng(1).standard_normal((E, H)).astype(np.float32)
    x = np.zeros((H + 1, H))
    x[np.arange(H), np.arange(H)] = 1.0
    x[H] = 1.0
    l32, l64 = oracle.router_logits(x, wr)
    assert np.array_equal(l32[:H], wr.T)
    assert np.allclose(l64[H], wr.astype(np.float64).sum(axis=1), rtol=0, atol=1e-12)


def test_router_logits_brute_force_loop():
    x = np.random.default_rng(2).standard_normal((5, 40))
    wr = np.random.default_rng(3).standard_normal((8, 40)).astype(np.float32)
    _, l64 = oracle.router_logits(x, wr)
    for t in range(5):
        for e in range(8):
            s = 0.0
            for h in range(40):
                s += x[t, h] * float(wr[e, h])
            assert abs(s - l64[t, e]) < 1e-12


def test_uniform_routing_statistics_tiny_config():
    # x ~ N(0,1), Wr ~ N(0,1/H): logits ~ N(0,1); routing is near uniform
    cfg = synth.get_config("tiny").with_(T=4096)
    inp = synth.generate_host(cfg)
    l32, l64 = oracle.router_logits(oracle.widen(inp.x, cfg.act), inp.wr)
    assert 0.8 < l64.std() < 1.2
    r = oracle.top_k_softmax(l32, l64, 2)
    util = oracle.expert_utilization(r.idx, 8)
    assert np.all(np.abs(util - 1.0) < 0.3)
    assert abs(util.mean() - 1.0) < 1e-12
