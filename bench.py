"""Benchmark of the top-2 MoE FFN layer (Grok-1 shape) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload decode|prefill|skew|capacity|decode_i4|medium]

A step is one moe_layer_forward call: router + top-2 + softmax, dispatch,
gate/up GEMM with SwiGLU, down GEMM and combine, over one batch of seeded
synthetic inputs already resident in HBM. W untimed steps, then K steps
timed with HIP events between two device synchronisations. Prints ONE JSON
line on stdout (logs go to stderr):
  value      tokens/s of the whole layer at the chosen workload (default:
             the Grok-1-shape decode batch, T = 8);
  roofline   the dominant kernel (the gate/up GEMM: 2/3 of the flops and of
             the weight bytes) against HBM bandwidth or bf16 MFMA peak, by
             its arithmetic intensity: algorithmic bytes or flops per launch
             over the mean duration of K launches run back to back;
  layer      the whole layer's HBM and MFMA fractions, the median of single
             timed calls, per-GEMM times and the router's time;
  prefill, medium, decode_i4
             the same measurement at T = 8192 (one full context, MFMA-bound),
             T = 512 (one 512-token sequence, about 128 rows per expert) and
             with int4 weights at T = 8;
  train      a training step on the same weights at T = 8192 with capacity
             1.25: moe_layer_forward_train + moe_layer_backward, tokens/s,
             stage times and the weight-gradient GEMM against bf16 MFMA peak;
  cpu_baseline  the oracle (numpy float64, test infrastructure) on a bounded
             sample of the same workload on this host's cores; the prefill
             line carries its own (routing over all tokens, the expert FFN on
             256 sampled tokens, the full layer time extrapolated).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MoE-layer tokens/sec at Grok-1 shape; % HBM BW (decode) / % MFMA peak (prefill)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gateup_decode": ["sparse_moe_transformer_top_amd/csrc/ffn_decode.hip",
                      "sparse_moe_transformer_top_amd/csrc/ffn_decode_lds.hip",
                      "sparse_moe_transformer_top_amd/csrc/common.h"],
    "gateup_tiled": ["sparse_moe_transformer_top_amd/csrc/ffn_tiled.hip",
                     "sparse_moe_transformer_top_amd/csrc/common.h",
                     "sparse_moe_transformer_top_amd/csrc/grouped.h"],
    "wgrad": ["sparse_moe_transformer_top_amd/csrc/ffn_tiled.hip",
              "sparse_moe_transformer_top_amd/csrc/common.h",
              "sparse_moe_transformer_top_amd/csrc/grouped.h"],
}


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel calibration), if recorded for the
    current source of the kernel; None otherwise."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(f"{kernel}/{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


class Layer:
    """Inputs, workspace and the step functions of one workload."""

    def __init__(self, cfg, dev, torch, moe, weights=None):
        from synth.device import generate_device
        self.cfg, self.torch, self.moe = cfg, torch, moe
        if weights is None:
            self.d = generate_device(cfg, dev)
        else:
            xd = generate_device(cfg, dev, x_only=True)
            self.d = weights
            self.d = type(weights)(cfg, xd.x, xd.wr, weights.wg, weights.wu, weights.wd,
                                   weights.sg, weights.su, weights.sd)
        d = self.d
        self.ws = torch.empty(moe.layer_workspace_bytes(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k,
                                                        d.x.dtype, d.wg.dtype),
                              dtype=torch.uint8, device=dev)
        self.out = torch.empty((cfg.T, cfg.H), dtype=d.x.dtype, device=dev)

    def step(self):
        d, c = self.d, self.cfg
        self.moe.moe_layer_forward(d.x, d.wr, d.wg, d.wu, d.wd, k=c.k,
                                   capacity_factor=c.capacity_factor, s_gate=d.sg, s_up=d.su,
                                   s_down=d.sd, workspace=self.ws, out=self.out)

    def per_call_ms(self, steps):
        """Durations of `steps` single layer calls, each between its own pair
        of events on the library's stream (torch's current stream)."""
        torch = self.torch
        evs = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            self.step()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    def timed(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            self.step()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def kernel_times(self, reps):
        """Mean duration (ms) of the gate/up and of the down launches: the
        layer's routing and dispatch are made once, then `reps` launches of
        each GEMM run back to back (moe_expert_gate_up, moe_expert_down into
        the same buffers), queued behind a ~2 ms device-side delay so that the
        events on the library's stream bracket the kernels and not the host's
        launch latency. Returns (gate/up ms, down ms, dispatch)."""
        torch, d, c, m = self.torch, self.d, self.cfg, self.moe
        idx, w = m.moe_router_topk(d.x, d.wr, c.k)
        disp = m.moe_dispatch(idx, c.E, c.capacity_factor)
        h = m.moe_expert_gate_up(d.x, disp["perm"], disp["offsets"], c.k, d.wg, d.wu, d.sg, d.su)
        y = m.moe_expert_down(h, disp["offsets"], c.T, c.k, d.wd, d.sd)
        torch.cuda.synchronize()
        out = []
        for fn in (lambda: m.moe_expert_gate_up(d.x, disp["perm"], disp["offsets"], c.k, d.wg,
                                                d.wu, d.sg, d.su, h=h),
                   lambda: m.moe_expert_down(h, disp["offsets"], c.T, c.k, d.wd, d.sd,
                                             y_perm=y)):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(2_000_000)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / reps)
        return out[0], out[1], disp

    def router_time(self, reps=50):
        """Mean duration (ms) of moe_router_topk, back to back behind a delay."""
        torch, d, c, m = self.torch, self.d, self.cfg, self.moe
        idx, w = m.moe_router_topk(d.x, d.wr, c.k)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(2_000_000)
        a.record()
        for _ in range(reps):
            m.moe_router_topk(d.x, d.wr, c.k)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def routing_stats_time(self, reps=50):
        """Mean duration of moe_routing_stats on this workload's router
        logits and dispatch counts. The launches are queued behind a ~1 ms
        device-side delay (torch.cuda._sleep), so the events bracket
        back-to-back kernels rather than the host's launch latency."""
        torch, d, c, m = self.torch, self.d, self.cfg, self.moe
        idx, _, logits = m.moe_router_topk(d.x, d.wr, c.k, return_logits=True)
        counts = m.moe_dispatch(idx, c.E, c.capacity_factor)["counts"]
        for _ in range(3):
            m.moe_routing_stats(logits, counts, c.k)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(2_000_000)
        a.record()
        for _ in range(reps):
            m.moe_routing_stats(logits, counts, c.k)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps


    def ep_layout_time(self, R, reps=20):
        """Mean durations (ms) of moe_ep_pack and moe_ep_unpack for this
        workload's dispatch with the E experts on R ranks, the rows of all
        ranks' receive buffers handled on this GPU (pack: every kept row read
        and written once; unpack the same), queued behind a device-side delay."""
        torch, d, c, m = self.torch, self.d, self.cfg, self.moe
        idx, _ = m.moe_router_topk(d.x, d.wr, c.k)
        disp = m.moe_dispatch(idx, c.E, c.capacity_factor)
        send, cnt = m.moe_ep_pack(d.x, disp["perm"], disp["offsets"], c.k, R)
        n = int(disp["offsets"][-1].item())
        # one receive buffer holding everything: R x E/R counts from this dispatch
        rc = torch.diff(disp["offsets"]).view(1, c.E).to(torch.int32).contiguous()
        off, ridx = m.moe_ep_recv_layout(rc, n)
        y = send[:n]
        out = []
        for fn in (lambda: m.moe_ep_pack(d.x, disp["perm"], disp["offsets"], c.k, R),
                   lambda: m.moe_ep_unpack(y, ridx, off, n)):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(2_000_000)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / reps)
        return out[0], out[1], n


class TrainStep:
    """One training step of the layer: moe_layer_forward_train, then
    moe_layer_backward for a seeded output gradient, on the given weights."""

    def __init__(self, cfg, dev, torch, moe, weights):
        from synth.device import generate_device, grad_output_device
        self.cfg, self.torch, self.moe = cfg, torch, moe
        xd = generate_device(cfg, dev, x_only=True)
        self.d = type(weights)(cfg, xd.x, xd.wr, weights.wg, weights.wu, weights.wd,
                               None, None, None)
        T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
        self.dout = grad_output_device(T, H, seed=cfg.seed, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.res = torch.empty(moe.train_reserve_bytes(T, H, F, E, k), **u8)
        self.ws = torch.empty(moe.backward_workspace_bytes(T, H, F, E, k), **u8)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        d = self.d
        self.grads = dict(dx=torch.empty_like(d.x),
                          dw_router=torch.empty((E, H), dtype=torch.float32, device=dev),
                          dw_gate=torch.empty_like(d.wg), dw_up=torch.empty_like(d.wu),
                          dw_down=torch.empty_like(d.wd))

    def forward(self):
        d, c = self.d, self.cfg
        self.moe.moe_layer_forward_train(d.x, d.wr, d.wg, d.wu, d.wd, k=c.k,
                                         capacity_factor=c.capacity_factor, reserve=self.res,
                                         out=self.out)

    def backward(self, split=False):
        d, c = self.d, self.cfg
        self.moe.moe_layer_backward(d.x, d.wr, d.wg, d.wu, d.wd, self.dout, self.res, k=c.k,
                                    workspace=self.ws, grads=self.grads, split=split)

    def timed(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.forward()
            self.backward()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            self.forward()
            self.backward()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def stage_times(self, steps):
        """Mean ms of the forward, the backward's data step and its weight
        step (the two launches of the weight-gradient GEMM), with events
        between the calls on torch's current stream (the library's stream)."""
        torch, moe, d, c = self.torch, self.moe, self.d, self.cfg
        evs = []
        for _ in range(steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
            self.forward()
            ev[1].record()
            moe.moe_layer_backward(d.x, d.wr, d.wg, d.wu, d.wd, self.dout, self.res, k=c.k,
                                   workspace=self.ws, grads=self.grads, split=True)
            ev[2].record()
            evs.append(ev)
        torch.cuda.synchronize()
        fw = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        bw = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
        # the weight step on its own, behind a device-side delay so that the
        # events bracket the two GEMM launches and not the host
        wt = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(2_000_000)
            a.record()
            self.weights_step()
            b.record()
            torch.cuda.synchronize()
            wt.append(a.elapsed_time(b))
        return fw, bw, sum(wt) / steps

    def weights_step(self):
        c = self.cfg
        self.moe.moe_layer_backward_weights(self.res, self.ws, self.grads, c.T, c.H, c.F, c.E,
                                            c.k)

    def kept_rows(self):
        v = self.moe.train_reserve_views(self.res, self.cfg.T, self.cfg.H, self.cfg.F,
                                         self.cfg.E, self.cfg.k)
        return int(v["offsets"][-1].item())


def host_inputs(layer):
    """Host copies (storage form) of a workload's inputs for the oracle."""
    import numpy as np
    import torch

    def host_array(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
            else t.numpy()

    d, c = layer.d, layer.cfg
    return dict(x=host_array(d.x), wr=host_array(d.wr),
                wg=[host_array(d.wg[e]) for e in range(c.E)],
                wu=[host_array(d.wu[e]) for e in range(c.E)],
                wd=[host_array(d.wd[e]) for e in range(c.E)],
                **{n: (None if getattr(d, n) is None else host_array(getattr(d, n)))
                   for n in ("sg", "su", "sd")})


def host_inputs_x(layer):
    """Host copies of a workload's x and router weight (its expert weights are
    another workload's)."""
    import numpy as np
    import torch
    x = layer.d.x.detach().cpu().contiguous()
    x = x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()
    return dict(x=x, wr=layer.d.wr.detach().cpu().numpy())


def host_cores():
    """Host cores this process may run on, and the oracle's BLAS threads."""
    from threadpoolctl import threadpool_info
    cores = len(os.sched_getaffinity(0))
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return cores, int(blas)


def cpu_baseline(layer, h, n_tokens):
    """The oracle (numpy, float64 throughout, as it stands) on the first
    n_tokens tokens of the workload: routing and dispatch over all T tokens,
    expert FFN and combine for the sample."""
    import numpy as np
    import oracle
    c = layer.cfg
    tokens = np.arange(n_tokens)
    t0 = time.perf_counter()
    oracle.layer_forward(h["x"], c.act, h["wr"], h["wg"], h["wu"], h["wd"], c.wdt, k=c.k,
                         capacity_factor=c.capacity_factor, sg=h["sg"], su=h["su"],
                         sd=h["sd"], tokens=tokens)
    dt = time.perf_counter() - t0
    cores, blas = host_cores()
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": cores, "blas_threads": blas,
            "kind": "oracle", "precision": "float64", "seconds": round(dt, 2),
            "sample": (f"first {n_tokens} of the {c.T} tokens of the {c.name} workload: router, "
                       f"top-k and dispatch over all {c.T} tokens, expert FFN and combine for the "
                       f"sample (the oracle as it stands: numpy float64, OpenBLAS)")}


def cpu_baseline_sampled(layer, h, n_sample=256):
    """The oracle at a token count it cannot run whole in seconds: routing and
    dispatch over all T tokens (timed), the expert FFN and combine on a seeded
    sample of n_sample tokens (timed); tokens/s = n_sample / FFN time, and the
    full layer time extrapolated as routing + FFN time * T / n_sample."""
    import numpy as np
    import oracle
    c = layer.cfg
    sample = np.sort(np.random.default_rng(1).choice(c.T, n_sample, replace=False))
    t0 = time.perf_counter()
    x64 = oracle.widen(h["x"], c.act)
    l32, l64 = oracle.router_logits(x64, h["wr"])
    r = oracle.top_k_softmax(l32, l64, c.k)
    oracle.dispatch(r.idx, c.E, c.capacity_factor)
    t_route = time.perf_counter() - t0
    t1 = time.perf_counter()
    oracle.layer_forward(h["x"], c.act, h["wr"], h["wg"], h["wu"], h["wd"], c.wdt, k=c.k,
                         capacity_factor=c.capacity_factor, sg=h["sg"], su=h["su"],
                         sd=h["sd"], tokens=sample)
    t_all = time.perf_counter() - t1
    # layer_forward repeats the routing and dispatch over all T tokens
    t_ffn = max(t_all - t_route, 1e-9)
    cores, blas = host_cores()
    return {"value": n_sample / t_ffn, "unit": "tokens/s", "cores": cores,
            "blas_threads": blas, "kind": "oracle", "precision": "float64",
            "routing_dispatch_s": round(t_route, 2), "ffn_sample_s": round(t_ffn, 2),
            "extrapolated_layer_s": round(t_route + t_ffn * c.T / n_sample, 1),
            "sample": (f"{c.name} workload (T={c.T}): routing, top-k and dispatch over all "
                       f"{c.T} tokens; expert FFN and combine on a seeded sample of {n_sample} "
                       f"tokens (numpy default_rng(1)); value = sample / FFN time; the full "
                       f"layer time is extrapolated, not measured")}


def touched_experts(disp, E):
    off = disp["offsets"].cpu().tolist()
    n = [off[e + 1] - off[e] for e in range(E)]
    return sum(1 for v in n if v > 0), n, off[E]


RIDGE_FLOP_PER_BYTE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # 312.5


def roofline(kernel, algo_bytes, algo_flops, ms, traffic):
    """The kernel against the roof its arithmetic intensity puts it under:
    HBM below the ridge point (algorithmic bytes / time), bf16 MFMA above it
    (algorithmic flops / time)."""
    hbm = algo_flops / algo_bytes < RIDGE_FLOP_PER_BYTE
    if hbm:
        ach = algo_bytes / (ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = algo_flops / (ms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
    r.update({"traffic": traffic, "kernel": kernel, "algorithmic_bytes": int(algo_bytes),
              "algorithmic_flops": float(algo_flops), "mean_ms": round(ms, 4)})
    return r


def gateup_kernel_name(cfg):
    if cfg.T > 16:
        tiles = ("stream tiles for experts with <= 128 rows, wide tiles for the rest"
                 if cfg.T * cfg.k <= cfg.E * 256 else "wide tiles")
        return "ffn_mfma_kernel gate/up (%s weights; %s)" % (
            {"bf16": "bf16", "i8": "int8"}[cfg.wdt], tiles)
    if cfg.wdt == "bf16" and cfg.T <= 8:
        return "gateup_xlds_kernel (bf16 weights, token rows in LDS)"
    if cfg.wdt == "i4":
        return "gateup_decode_i4_kernel (int4 weights, 4 column tiles per work-group)"
    return "gateup_decode_kernel (%s weights)" % {"bf16": "bf16", "i8": "int8"}[cfg.wdt]


def measure(layer, steps, warmup):
    """One workload: the layer timed over `steps` calls between two
    synchronisations (after `warmup`), the median of single timed calls, and
    the gate/up GEMM (the dominant kernel: 2/3 of the flops and weight bytes)
    against its roof."""
    import statistics
    cfg = layer.cfg
    ms = layer.timed(steps, warmup)
    med = statistics.median(layer.per_call_ms(steps))
    gu_ms, dn_ms, disp = layer.kernel_times(steps)
    n_touched, n_per_e, n_kept = touched_experts(disp, cfg.E)
    esz = {"f32": 4, "bf16": 2, "i8": 1, "i4": 0.5}[cfg.wdt]
    asz = 2 if cfg.act == "bf16" else 4
    H, F = cfg.H, cfg.F
    # algorithmic work of the gate/up launch: every touched expert's gate and
    # up weights read once (+ scales: int8 one float32 per weight row, int4
    # one per row and 128 k), the gathered x rows read, h written
    gu_scales = {"i8": 2 * F * 4, "i4": 2 * F * (H // 128) * 4}.get(cfg.wdt, 0)
    dn_scales = {"i8": H * 4, "i4": H * (F // 128) * 4}.get(cfg.wdt, 0)
    gu_bytes = int(n_touched * 2 * F * H * esz) + n_kept * (H + F) * asz + n_touched * gu_scales
    gu_flops = 4.0 * H * F * n_kept
    # whole layer: every touched expert's three matrices once, x read and out
    # written, h and y_perm each written once and read once
    layer_bytes = int(n_touched * 3 * F * H * esz) + cfg.T * H * asz * 2 + \
        n_kept * (H + F) * asz * 2 + n_touched * (gu_scales + dn_scales)
    layer_flops = 6.0 * H * F * n_kept
    kind = "gateup_decode" if cfg.T <= 16 else "gateup_tiled"
    roof = roofline(gateup_kernel_name(cfg), gu_bytes, gu_flops, gu_ms,
                    traffic_from_profiles(kind, cfg.name))
    lay = {"hbm_GBps": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
           "hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "TFLOPs": round(layer_flops / (ms * 1e-3) / 1e12, 2),
           "mfma_frac": round(layer_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "median_ms_per_call": round(med, 4),
           "stages_ms": {"gate_up": round(gu_ms, 4), "down": round(dn_ms, 4)}}
    info = {"experts_touched": n_touched, "rows_per_expert": n_per_e, "kept": n_kept}
    return ms, roof, lay, info


def secondary(layer, steps, warmup):
    """A compact line for a secondary workload."""
    ms, roof, lay, info = measure(layer, steps, warmup)
    cfg = layer.cfg
    return {"workload": f"{cfg.name}: {cfg.description}", "T": cfg.T, "weights": cfg.wdt,
            "tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "roofline": roof, "layer": lay, **info}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "skew", "capacity", "decode_i4", "medium"])
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary lines (prefill, medium, int4 decode, training step)")
    ap.add_argument("--no-train", action="store_true", help="skip the training-step secondary line")
    ap.add_argument("--cpu-tokens", type=int, default=8,
                    help="tokens in the oracle's timed sample at decode sizes (0 skips the CPU "
                         "baselines); workloads above 16 tokens time a 256-token sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (float32 negate: reads "
                         "and writes MIB MiB per launch) 3 times, to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20 // 4
        a = torch.randn(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n * 4}))
        return
    import synth
    import sparse_moe_transformer_top_amd as moe
    moe.load_library()
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.workload]
    log(f"generating {cfg.name}: T={cfg.T} H={cfg.H} F={cfg.F} E={cfg.E} k={cfg.k} "
        f"{cfg.act}/{cfg.wdt} cf={cfg.capacity_factor}")
    layer = Layer(cfg, dev, torch, moe)
    torch.cuda.synchronize()

    ms, roof, lay, info = measure(layer, args.steps, args.warmup)
    log(f"{cfg.name}: {ms:.4f} ms/step (median single call {lay['median_ms_per_call']:.4f} ms)")
    result = {
        "metric": METRIC, "value": round(cfg.T / (ms * 1e-3), 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.act if cfg.wdt in ("f32", "bf16") else
                 "bf16 (%s weights)" % {"i8": "int8", "i4": "int4"}[cfg.wdt], "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "T": cfg.T, "H": cfg.H,
                   "F": cfg.F, "E": cfg.E, "k": cfg.k, "capacity_factor": cfg.capacity_factor,
                   "weights": cfg.wdt, "experts_touched": info["experts_touched"],
                   "rows_per_expert": info["rows_per_expert"]},
        "roofline": roof,
        "layer": lay,
    }
    result["layer"]["router_us"] = round(layer.router_time() * 1e3, 2)

    # routing statistics (per-token margin and outside-top-k mass, per-expert
    # utilisation): reads the T x E float32 logits and the counts, writes 8
    # bytes per token and 4 per expert
    rs_ms = layer.routing_stats_time()
    rs_bytes = cfg.T * cfg.E * 4 + cfg.T * 8 + cfg.E * 8
    result["routing_stats"] = {"us": round(rs_ms * 1e3, 2), "bytes": rs_bytes,
                               "GBps": round(rs_bytes / (rs_ms * 1e-3) / 1e9, 1)}

    # expert-parallel layouts (E experts on E ranks): pack and unpack each read
    # and write every kept row once
    asz = 2 if cfg.act == "bf16" else 4
    pk_ms, up_ms, n_rows = layer.ep_layout_time(cfg.E)
    ep_bytes = 2 * n_rows * cfg.H * asz
    result["ep_layout"] = {"ranks": cfg.E, "rows": n_rows,
                           "pack_us": round(pk_ms * 1e3, 2),
                           "pack_GBps": round(ep_bytes / (pk_ms * 1e-3) / 1e9, 1),
                           "unpack_us": round(up_ms * 1e3, 2),
                           "unpack_GBps": round(ep_bytes / (up_ms * 1e-3) / 1e9, 1)}

    pl = None
    if not args.no_secondary and cfg.name == "decode":
        sub = max(5, args.steps // 2)
        for name in ("prefill", "medium"):
            log(f"{name} secondary line: same weights, T={synth.CONFIGS[name].T} tokens")
            sl = Layer(synth.CONFIGS[name], dev, torch, moe, weights=layer.d)
            result[name] = secondary(sl, sub, 2)
            result[name]["router_us"] = round(sl.router_time() * 1e3, 2)
            if name == "prefill":
                ppk, pup, prows = sl.ep_layout_time(sl.cfg.E)
                pbytes = 2 * prows * cfg.H * 2
                result[name]["ep_layout"] = {
                    "ranks": sl.cfg.E, "rows": prows, "pack_us": round(ppk * 1e3, 1),
                    "pack_GBps": round(pbytes / (ppk * 1e-3) / 1e9, 1),
                    "unpack_us": round(pup * 1e3, 1),
                    "unpack_GBps": round(pbytes / (pup * 1e-3) / 1e9, 1)}
                pl = sl
            else:
                del sl
        log("decode_i4 secondary line: int4 weights, T=8 tokens")
        il = Layer(synth.CONFIGS["decode_i4"], dev, torch, moe)
        result["decode_i4"] = secondary(il, args.steps, args.warmup)
        del il
        torch.cuda.empty_cache()

    if not args.no_secondary and not args.no_train and cfg.name == "decode":
        tcfg = synth.CONFIGS["train"]
        log("training step: same weights, T=8192 tokens, capacity 1.25")
        tr = TrainStep(tcfg, dev, torch, moe, layer.d)
        nsteps = max(3, args.steps // 4)
        tms = tr.timed(nsteps, 2)
        fw, bw, wt = tr.stage_times(nsteps)
        nk = tr.kept_rows()
        H, F = cfg.H, cfg.F
        # flops: forward 6 n H F; backward 12 n H F (dh 2, dx 4, dW_down 2,
        # dW_gate|dW_up 4); the weight step's two launches hold 6 n H F
        tflops = 18.0 * H * F * nk
        wflops = 6.0 * H * F * nk
        wach = wflops / (wt * 1e-3) / 1e12
        result["train"] = {
            "workload": f"train: {tcfg.description}", "tokens_per_s": round(tcfg.T / (tms * 1e-3), 1),
            "ms_per_step": round(tms, 3), "kept_rows": nk,
            "TFLOPs": round(tflops / (tms * 1e-3) / 1e12, 1),
            "mfma_frac": round(tflops / (tms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "stages_ms": {"forward_train": round(fw, 3), "backward": round(bw, 3),
                          "backward_weights": round(wt, 3)},
            "roofline": {"bound": "mfma", "kernel": "wgrad_tn_kernel (dW_down, then "
                         "dW_gate|dW_up: 2 launches per step)",
                         "achieved": round(wach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(wach / BF16_PEAK_TFLOPS, 4),
                         "algorithmic_flops": wflops / 2, "mean_ms": round(wt / 2, 4),
                         "traffic": traffic_from_profiles("wgrad", "train")}}
        del tr
        torch.cuda.empty_cache()

    if args.cpu_tokens > 0:
        log("cpu baselines: copying the inputs to the host")
        h = host_inputs(layer)
        if cfg.T > 16:
            # MFMA-bound workloads: routing and dispatch over all T, the FFN
            # on a 256-token sample, the full layer extrapolated
            log(f"cpu baseline of the {cfg.name} workload (256-token sample)")
            result["cpu_baseline"] = cpu_baseline_sampled(layer, h)
        else:
            result["cpu_baseline"] = cpu_baseline(layer, h, min(args.cpu_tokens, cfg.T))
        if pl is not None:
            hp = dict(h)
            hx = host_inputs_x(pl)
            hp.update(hx)
            log("cpu baseline of the prefill workload (256-token sample)")
            result["prefill"]["cpu_baseline"] = cpu_baseline_sampled(pl, hp)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
