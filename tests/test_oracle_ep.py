"""Pins of the oracle's expert-parallel layouts (CPU only): a hand case of
the receive layout, and the whole EP data path on R emulated ranks (pack,
exchange by slicing, receive layout, local experts, unpack, return exchange,
combine) giving the single-device layer's output."""
import numpy as np
import pytest

import oracle
import synth


def test_recv_layout_hand_case():
    # two sources, two local experts: source 0 sends 1 row for e0 and 2 for e1,
    # source 1 sends 3 for e0 and none for e1; the buffer is p0e0 | p0e1 | p1e0
    off, idx = oracle.ep_recv_layout(np.array([[1, 2], [3, 0]]))
    assert off.tolist() == [0, 4, 6]
    assert idx.tolist() == [0, 3, 4, 5, 1, 2]
    back = oracle.ep_unpack(np.arange(6)[:, None] * 10.0, idx, 6)
    assert back[:, 0].tolist() == [0.0, 40.0, 50.0, 10.0, 20.0, 30.0]


def test_pack_counts_and_rows():
    rng = np.random.default_rng(2)
    T, E, k, H = 40, 8, 2, 4
    x = rng.standard_normal((T, H))
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    d = oracle.dispatch(idx, E, 1.0)           # with drops
    for R in (1, 2, 4, 8):
        rows, cnt = oracle.ep_pack(x, d.perm, d.offsets, k, E, R)
        assert cnt.sum() == d.offsets[E] == rows.shape[0]
        # every kept assignment's token row appears once, in dispatch order
        kept = [a for a in range(T * k) if d.slot_row[a] >= 0]
        assert sorted(d.perm[:d.offsets[E]].tolist()) == sorted(kept)
        for j in range(rows.shape[0]):
            assert np.array_equal(rows[j], x[d.perm[j] // k])
    with pytest.raises(ValueError):
        oracle.ep_pack(x, d.perm, d.offsets, k, E, 3)


@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_ep_path_equals_single_device_layer(R):
    cfg = synth.get_config("p_bf16").with_(T=90)
    inp = synth.generate_host(cfg)
    E, k, El = cfg.E, cfg.k, cfg.E // R
    x64 = oracle.widen(inp.x, cfg.act)
    wg = [oracle.widen(inp.wg[e], cfg.wdt) for e in range(E)]
    wu = [oracle.widen(inp.wu[e], cfg.wdt) for e in range(E)]
    wd = [oracle.widen(inp.wd[e], cfg.wdt) for e in range(E)]
    # tokens split unevenly over the R ranks
    cuts = np.linspace(0, cfg.T, R + 1).astype(int)
    cuts[1:-1] += np.arange(1, R) % 3
    ranks = []
    for p in range(R):
        xs = inp.x[cuts[p]:cuts[p + 1]]
        l32, l64 = oracle.router_logits(oracle.widen(xs, cfg.act), inp.wr)
        ro = oracle.top_k_softmax(l32, l64, k)
        d = oracle.dispatch(ro.idx, E, None)
        rows, cnt = oracle.ep_pack(oracle.widen(xs, cfg.act), d.perm, d.offsets, k, E, R)
        ranks.append((xs, ro, d, rows, cnt))
    # exchange: destination r receives, from each source p, the rows of its experts
    back_to = {p: [] for p in range(R)}
    for r in range(R):
        recv, rc = [], np.zeros((R, El), np.int64)
        for p, (_, _, d, rows, cnt) in enumerate(ranks):
            s0 = int(cnt[:r].sum())
            recv.append(rows[s0:s0 + cnt[r]])
            rc[p] = np.diff(d.offsets)[r * El:(r + 1) * El]
        recv = np.concatenate(recv)
        off, idx = oracle.ep_recv_layout(rc)
        y = np.zeros_like(recv)
        for e in range(El):
            seg = idx[off[e]:off[e + 1]]
            if len(seg):
                g = r * El + e
                y[off[e]:off[e + 1]] = oracle.swiglu_expert(recv[seg], wg[g], wu[g], wd[g])
        back = oracle.ep_unpack(y, idx, recv.shape[0])
        # return exchange: source p's block of this destination's buffer
        pos = 0
        for p in range(R):
            n = int(rc[p].sum())
            back_to[p].append(back[pos:pos + n])
            pos += n
    for p, (xs, ro, d, rows, cnt) in enumerate(ranks):
        y_perm = np.concatenate(back_to[p])           # the source's dispatch order
        out = oracle.combine(y_perm, d.slot_row, ro.w)
        ref = oracle.layer_forward(xs, cfg.act, inp.wr, inp.wg, inp.wu, inp.wd, cfg.wdt, k=k)
        assert np.allclose(out, ref.out, rtol=0, atol=1e-12 * max(1.0, np.abs(ref.out).max()))
