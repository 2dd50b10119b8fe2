"""Layer calls in flight on two streams at once (default priority), each with
its own workspace and output: the library keeps no state between calls, so
every result equals, bitwise, the same call made alone. Covers the decode
kernels and the tiled MFMA kernels (whose split tail tiles use the
workspace's scratch), with and without a capacity limit."""
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


@pytest.mark.parametrize("names", [("p_bf16", "p_cap"), ("p_bf16_dec", "p_bf16"),
                                   ("p_cap", "p_cap")])
def test_two_streams_match_sequential_calls(moe, names):
    cfgs = [synth.get_config(n).with_(seed=synth.get_config(n).seed + 10 * i)
            for i, n in enumerate(names)]
    log(f"two streams: {names}")
    ds = [to_device(synth.generate_host(c)) for c in cfgs]

    def call(c, d, ws=None, out=None):
        return moe.moe_layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], k=c.k,
                                     capacity_factor=c.capacity_factor, workspace=ws, out=out)

    # each call alone, one after the other
    ref = []
    for c, d in zip(cfgs, ds):
        ref.append(call(c, d).clone())
        torch.cuda.synchronize()
    wss = [torch.empty(moe.layer_workspace_bytes(c.T, c.H, c.F, c.E, c.k, d["x"].dtype,
                                                 d["wg"].dtype), dtype=torch.uint8, device="cuda")
           for c, d in zip(cfgs, ds)]
    outs = [torch.empty_like(d["x"]) for d in ds]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        # interleave the launches: each stream gets its call twice in a row
        for _ in range(2):
            for s, c, d, ws, out in zip(streams, cfgs, ds, wss, outs):
                with torch.cuda.stream(s):
                    call(c, d, ws, out)
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(2):
            assert _same(outs[i], ref[i]), (names, i, rep)
