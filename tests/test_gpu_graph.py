"""The layer forward inside a captured HIP graph (torch.cuda.graph): replays
with new inputs written into the captured buffers between them, and eager
work on the same stream in between, each equal bitwise to an eager call on
the same inputs. Covers the decode kernels (T <= 16, token rows staged in
LDS) and the tiled MFMA kernels, with and without a capacity limit, and the
matrix-core router."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_transformer_top_amd as m
    m.load_library()
    return m


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


# the last case routes on the matrix-core router kernel (from 4608 tokens)
GRAPH_CASES = ["p_dec1", "p_bf16_dec", "p_bf16", "p_cap", "many_tokens"]


def _graph_config(name):
    if name == "many_tokens":
        return synth.LayerConfig("g_many_tokens", T=4700, H=512, F=256, capacity_factor=1.25,
                                 seed=21)
    cfg = synth.get_config(name)
    return cfg.with_(T=8) if cfg.T < 8 else cfg


@pytest.mark.parametrize("name", GRAPH_CASES)
def test_layer_forward_graph_replays(moe, name):
    cfg = _graph_config(name)
    log(f"graph capture {name}: T={cfg.T} cf={cfg.capacity_factor}")
    d = to_device(synth.generate_host(cfg))
    x = d["x"].clone()
    ws = torch.empty(moe.layer_workspace_bytes(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, x.dtype,
                                               d["wg"].dtype), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    run = lambda: moe.moe_layer_forward(x, d["wr"], d["wg"], d["wu"], d["wd"], k=cfg.k,
                                        capacity_factor=cfg.capacity_factor, workspace=ws,
                                        out=out)
    # warm up on a side stream (first launches set kernel attributes), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    gen = torch.Generator(device="cuda")
    for rep in range(3):
        gen.manual_seed(100 + rep)
        x.copy_(torch.randn(x.shape, device="cuda", generator=gen).to(x.dtype))
        g.replay()
        got = out.clone()
        # eager work between replays, then the eager reference on the same x
        ref = moe.moe_layer_forward(x, d["wr"], d["wg"], d["wu"], d["wd"], k=cfg.k,
                                    capacity_factor=cfg.capacity_factor)
        torch.cuda.synchronize()
        assert _same(got, ref), f"replay {rep} differs from the eager call"


def test_training_step_graph_replays(moe):
    cfg = synth.get_config("p_cap")
    log(f"graph capture of a training step: T={cfg.T} cf={cfg.capacity_factor}")
    d = to_device(synth.generate_host(cfg))
    T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    x = d["x"].clone()
    dout = torch.empty_like(x)
    res = torch.empty(moe.train_reserve_bytes(T, H, F, E, k), dtype=torch.uint8, device="cuda")
    ws = torch.empty(moe.backward_workspace_bytes(T, H, F, E, k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(x)
    grads = dict(dx=torch.empty_like(x), dw_router=torch.empty_like(d["wr"]),
                 dw_gate=torch.empty_like(d["wg"]), dw_up=torch.empty_like(d["wu"]),
                 dw_down=torch.empty_like(d["wd"]))

    def step():
        moe.moe_layer_forward_train(x, d["wr"], d["wg"], d["wu"], d["wd"], k=k,
                                    capacity_factor=cfg.capacity_factor, reserve=res, out=out)
        moe.moe_layer_backward(x, d["wr"], d["wg"], d["wu"], d["wd"], dout, res, k=k,
                               workspace=ws, grads=grads)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    gen = torch.Generator(device="cuda")
    for rep in range(3):
        gen.manual_seed(200 + rep)
        x.copy_(torch.randn(x.shape, device="cuda", generator=gen).to(x.dtype))
        dout.copy_(torch.randn(x.shape, device="cuda", generator=gen).to(x.dtype))
        g.replay()
        got = {n: t.clone() for n, t in grads.items()}
        got_out = out.clone()
        ref_out, ref_res = moe.moe_layer_forward_train(x, d["wr"], d["wg"], d["wu"], d["wd"], k=k,
                                                       capacity_factor=cfg.capacity_factor)
        ref = moe.moe_layer_backward(x, d["wr"], d["wg"], d["wu"], d["wd"], dout, ref_res, k=k)
        torch.cuda.synchronize()
        assert _same(got_out, ref_out), f"replay {rep}: out"
        for n in got:
            a, b = got[n], ref[n]
            same = _same(a, b) if a.dtype == torch.bfloat16 else torch.equal(a, b)
            assert same, f"replay {rep}: {n}"
