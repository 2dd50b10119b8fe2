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


# --- routing statistics (the page's post-training utilisation analysis and
# its remark on the gap to the 3rd expert) ---------------------------------

def test_routing_stats_hand_cases():
    l = np.array([[5.0, 1.0, 2.0, 0.0]], np.float32)
    c = np.zeros(4)
    assert oracle.routing_stats(l, 1, c).margin[0] == 3.0
    assert oracle.routing_stats(l, 2, c).margin[0] == 1.0
    assert oracle.routing_stats(l, 3, c).margin[0] == 1.0
    assert oracle.routing_stats(l, 4, c).margin[0] == np.inf
    assert oracle.routing_stats(l, 4, c).unselected_mass[0] == 0.0
    # ln 3 against three zeros, top-1: 3 / (3 + 3) outside-mass 1/2
    l = np.array([[math.log(3.0), 0.0, 0.0, 0.0]], np.float32)
    m = oracle.routing_stats(l, 1, c).unselected_mass[0]
    assert abs(m - 3.0 / (float(np.float32(3.0)) + 3.0)) < 1e-7
    # all equal: (E - k) / E outside the selection, margin 0 (tie at the boundary)
    r = oracle.routing_stats(np.zeros((3, 8), np.float32), 2, np.zeros(8))
    assert np.all(r.unselected_mass == 0.75) and np.all(r.margin == 0.0)


def test_routing_stats_two_level_closed_form():
    # k selected logits at a, E - k at b: outside mass (E-k) e^b / (k e^a + (E-k) e^b)
    for E, k, a, b in ((8, 2, 1.5, -0.25), (16, 4, 0.0, -3.0), (4, 1, 2.0, 2.0 - 1e-3)):
        l = np.full((1, E), b, np.float32)
        l[0, :k] = a
        r = oracle.routing_stats(l, k, np.zeros(E))
        a64, b64 = float(np.float32(a)), float(np.float32(b))
        want = (E - k) * math.exp(b64) / (k * math.exp(a64) + (E - k) * math.exp(b64))
        assert abs(r.unselected_mass[0] - want) < 1e-12
        assert r.margin[0] == a64 - b64


def test_routing_stats_brute_force():
    rng = np.random.default_rng(12)
    for E in (4, 8, 16):
        for k in range(1, min(E, 4) + 1):
            # integer logits force ties, including at the k / k+1 boundary
            l = np.where(rng.random((40, E)) < 0.5, rng.integers(-2, 3, (40, E)),
                         rng.standard_normal((40, E))).astype(np.float32)
            r = oracle.routing_stats(l, k, np.zeros(E))
            for t in range(40):
                ranked = sorted(((-float(v), i) for i, v in enumerate(l[t])))
                chosen = {i for _, i in ranked[:k]}
                vals = [-nv for nv, _ in ranked]
                want_m = vals[k - 1] - vals[k] if k < E else math.inf
                assert r.margin[t] == want_m
                zs = [math.exp(float(v) - vals[0]) for v in l[t]]
                want = sum(z for i, z in enumerate(zs) if i not in chosen) / sum(zs)
                assert abs(r.unselected_mass[t] - want) < 1e-12


def test_selected_weights_match_unselected_mass():
    # the softmax over the k selected logits is the full softmax renormalised
    # by what the selection holds: w_j = p_j / (1 - outside mass)
    rng = np.random.default_rng(5)
    l32 = rng.standard_normal((30, 8)).astype(np.float32)
    for k in (1, 2, 3):
        ro = oracle.top_k_softmax(l32, l32.astype(np.float64), k)
        st = oracle.routing_stats(l32, k, np.zeros(8))
        l = l32.astype(np.float64)
        p = np.exp(l - l.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        psel = np.take_along_axis(p, ro.idx.astype(np.int64), axis=1)
        assert np.allclose(ro.w * (1.0 - st.unselected_mass)[:, None], psel, rtol=0, atol=1e-14)


def test_utilization_from_dispatch_counts():
    # the dispatch's sequential counts give the same utilisation as a bincount
    # of the indices; it sums to E
    rng = np.random.default_rng(8)
    for E, k, T in ((8, 2, 500), (16, 4, 97), (4, 1, 33)):
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        counts = oracle.dispatch(idx, E, None).counts
        r = oracle.routing_stats(np.zeros((T, E), np.float32), k, counts)
        assert np.array_equal(r.utilization, oracle.expert_utilization(idx, E))
        assert abs(r.utilization.sum() - E) < 1e-12
    assert np.all(oracle.routing_stats(np.zeros((0, 8), np.float32), 2, np.zeros(8)).utilization == 0)
