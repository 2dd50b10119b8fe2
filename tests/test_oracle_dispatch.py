"""Pins of the oracle's dispatch and capacity drop (CPU only)."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_sizes.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        rows.setdefault(key, []).append([int(v) for v in vals])
    return rows


def _random_idx(T, E, k, seed, p=None):
    rng = np.random.default_rng(seed)
    idx = np.empty((T, k), np.int32)
    for t in range(T):
        idx[t] = rng.choice(E, size=k, replace=False, p=p)
    return idx


def _vectorised_ranks(idx, E):
    # independent formulation: one-hot [T,E] occupancy, exclusive cumsum down
    # the token axis gives each (token, expert) its number of earlier tokens
    T, k = idx.shape
    occ = np.zeros((T, E), np.int64)
    occ[np.repeat(np.arange(T), k), idx.ravel()] = 1
    excl = np.cumsum(occ, axis=0) - occ
    return excl[np.repeat(np.arange(T), k), idx.ravel()].reshape(T, k)


def _check_invariants(idx, E, d, cap):
    T, k = idx.shape
    N = T * k
    assert d.counts.sum() == N
    kept = d.counts if cap is None else np.minimum(d.counts, cap)
    assert np.array_equal(np.diff(d.offsets), kept)
    assert d.offsets[0] == 0 and d.offsets[E] == kept.sum()
    n_kept = int(d.offsets[E])
    drops = 0 if cap is None else int(np.maximum(d.counts - cap, 0).sum())
    assert int(d.dropped.sum()) == drops == N - n_kept
    assert np.all(d.perm[n_kept:] == -1)
    head = d.perm[:n_kept]
    assert len(np.unique(head)) == n_kept and head.min(initial=0) >= 0
    for a in range(N):
        r = d.slot_row[a]
        assert (r == -1) == bool(d.dropped[a])
        if r >= 0:
            assert d.perm[r] == a
    for e in range(E):
        rows = d.perm[d.offsets[e]:d.offsets[e + 1]]
        assert np.all(idx.ravel()[rows] == e)
        tok = rows // k
        assert np.all(np.diff(tok) > 0)    # ascending token order within an expert


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (37, 8, 2), (500, 8, 2), (64, 4, 3), (200, 16, 1)])
def test_no_capacity_invariants(T, E, k):
    idx = _random_idx(T, E, k, seed=T)
    d = oracle.dispatch(idx, E, None)
    assert d.cap is None
    _check_invariants(idx, E, d, None)
    # every token appears in exactly k rows with distinct experts
    tok = d.perm // k
    assert np.all(np.bincount(tok, minlength=T) == k)


@pytest.mark.parametrize("cf", [1.0, 1.25, 0.5])
def test_capacity_matches_vectorised_ranks(cf):
    T, E, k = 400, 8, 2
    p = np.array([0.4, 0.2, 0.1, 0.1, 0.05, 0.05, 0.05, 0.05])
    idx = _random_idx(T, E, k, seed=5, p=p)
    d = oracle.dispatch(idx, E, cf)
    cap = int(np.ceil(cf * T * k / E))
    assert d.cap == cap
    _check_invariants(idx, E, d, cap)
    rank = _vectorised_ranks(idx, E)
    assert np.array_equal(d.dropped.reshape(T, k).astype(bool), rank >= cap)
    off = d.offsets[idx]
    expect_row = np.where(rank < cap, off + rank, -1)
    assert np.array_equal(d.slot_row.reshape(T, k), expect_row)
    assert d.dropped.sum() > 0


def test_capacity_values():
    # ceil(1.25 * T * k / E): 5120 at T = 16384 (k = 2, E = 8)
    assert oracle.capacity(16384, 2, 8, 1.25) == 5120
    assert oracle.capacity(10, 2, 8, 1.25) == 4          # ceil(3.125)
    for cf in (None, 0.0, -1.0, float("inf")):
        assert oracle.capacity(100, 2, 8, cf) is None


def test_both_slots_dropped():
    # tokens 0..3 all choose experts (0,1); capacity 2 keeps tokens 0 and 1 only
    idx = np.array([[0, 1]] * 4, np.int32)
    d = oracle.dispatch(idx, 2, 1.0)      # cap = ceil(1.0 * 8 / 2) = 4? -> use E=2
    assert d.cap == 4
    d = oracle.dispatch(idx, 8, 1.0)      # cap = ceil(8/8) = 1
    assert d.cap == 1
    assert d.dropped.tolist() == [0, 0, 1, 1, 1, 1, 1, 1]
    assert d.counts.tolist() == [4, 4, 0, 0, 0, 0, 0, 0]
    assert d.offsets.tolist() == [0, 1, 2, 2, 2, 2, 2, 2, 2]
    assert d.perm.tolist() == [0, 1, -1, -1, -1, -1, -1, -1]


def test_empty_input():
    d = oracle.dispatch(np.zeros((0, 2), np.int32), 8, 1.25)
    assert d.counts.tolist() == [0] * 8 and d.offsets.tolist() == [0] * 9
    assert d.perm.size == 0 and d.slot_row.size == 0


def test_page_sizes_golden():
    g = _golden()
    H, F = g["hidden"][0][0], g["expert_dim"][0][0]
    E, k = g["num_experts"][0][0], g["top_k"][0][0]
    assert (H, F, E, k) == (6144, 32768, 8, 2)
    # fused gate/up is [2F, H] stored out x in, printed in x out
    assert g["w_gate_up_in_out"][0] == [H, 2 * F]
    assert g["w_down_in_out"][0] == [F, H]
    for b, s, per in g["expert_batch"]:
        assert oracle.mean_rows_per_expert(b * s, k, E) == per
        # the dispatch's mean rows per expert equals the printed figure when
        # all b*s tokens route without a drop
        assert b * s * k // E == per
    # all 8 experts of one layer in bf16: 3*H*F*2 B * 8 ~= 9.66 GB
    assert oracle.expert_params(H, F) * 2 * E == 9_663_676_416


def test_expert_utilization_normalisation():
    idx = np.array([[e, (e + 1) % 8] for e in range(8)] * 3, np.int32)
    u = oracle.expert_utilization(idx, 8)
    assert np.allclose(u, 1.0)
