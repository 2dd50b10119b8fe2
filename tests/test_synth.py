"""Checks of the seeded input generator (CPU only)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    a = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 3
    a[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # ties to even
    ours = synth.bf16_bits_from_f32(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.f32_from_bf16_bits(ours),
                          torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_int8_quantisation_rule():
    w = np.random.default_rng(1).standard_normal((50, 300)).astype(np.float32)
    q, s = synth.quantize_int8_rows(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.all(np.abs(q).max(axis=1) == 127)
    err = np.abs(q.astype(np.float64) * s[:, None] - w)
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-5))


def test_distributions_and_determinism():
    cfg = synth.get_config("tiny").with_(T=512, F=1024)
    a = synth.generate_host(cfg)
    b = synth.generate_host(cfg)
    for k, v in a.arrays().items():
        assert np.array_equal(v, b.arrays()[k]), k
    assert abs(a.x.std() - 1) < 0.02
    assert abs(a.wr.std() * np.sqrt(cfg.H) - 1) < 0.1
    assert abs(a.wg.std() * np.sqrt(cfg.H) - 1) < 0.02
    assert abs(a.wd.std() * np.sqrt(cfg.F) - 1) < 0.02


def test_storage_dtypes():
    for name, xt, wt in [("p_bf16", np.uint16, np.uint16), ("p_i8", np.uint16, np.int8),
                         ("p_f32", np.float32, np.float32)]:
        cfg = synth.get_config(name).with_(T=8)
        inp = synth.generate_host(cfg)
        assert inp.x.dtype == xt and inp.wg.dtype == wt and inp.wr.dtype == np.float32
        assert inp.wg.shape == (cfg.E, cfg.F, cfg.H) and inp.wd.shape == (cfg.E, cfg.H, cfg.F)
        if cfg.wdt == "i8":
            assert inp.sg.shape == (cfg.E, cfg.F) and inp.sd.shape == (cfg.E, cfg.H)


def _top1_shares(cfg, skew=None):
    import oracle
    x, wr = synth.router_inputs(cfg if skew is None else cfg.with_(skew=skew))
    l32, l64 = oracle.router_logits(oracle.widen(x, cfg.act), wr)
    return np.bincount(oracle.top_k_softmax(l32, l64, cfg.k).idx[:, 0], minlength=cfg.E) / cfg.T


def test_router_inputs_are_generate_hosts_draws():
    cfg = synth.get_config("p_skew")
    a = synth.generate_host(cfg)
    x, wr = synth.router_inputs(cfg)
    assert np.array_equal(a.x, x) and np.array_equal(a.wr, wr)


def test_skew_magnitudes_give_the_target_top1_shares():
    # The skewed workloads ask for about 50% / 25% of the top-1 picks on
    # experts 0 / 1; the stored magnitudes (along the mean direction of x)
    # were chosen on a 0.2 grid with the host draws of seed 0. At T = 4096
    # they reach the target within a percent and no neighbour on the grid is
    # closer; at T = 16384 the stored pair gives the closest shares the grid
    # reached (the second expert's share falls as the first's rises).
    cfg = synth.CONFIGS["skew"]
    a0, a1 = cfg.skew
    s = _top1_shares(cfg)
    assert abs(s[0] - 0.50) < 0.01 and abs(s[1] - 0.25) < 0.01, s[:2]
    dist = lambda v: (v[0] - 0.5) ** 2 + (v[1] - 0.25) ** 2
    for d0 in (-0.2, 0.0, 0.2):
        for d1 in (-0.2, 0.0, 0.2):
            if d0 or d1:
                assert dist(_top1_shares(cfg, (a0 + d0, a1 + d1))) >= dist(s) - 1e-12
    big = _top1_shares(synth.CONFIGS["capacity"])
    assert 0.46 < big[0] < 0.48 and 0.22 < big[1] < 0.23, big[:2]
