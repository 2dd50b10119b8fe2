"""GPU check of moe_layer_forward_noalloc (the layer forward on the library's
fixed scratch array) against moe_layer_forward with a caller workspace, through
the C ABI: the same kernels, so out and every routing output must be equal
bitwise. Each case makes two calls in a row on the shared scratch, the second
with fewer tokens, so that a result depending on what the first call left in
the array would show.
"""
import numpy as np
import pytest
import torch

import synth
from synth.device import generate_device
from gpu_helpers import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_transformer_top_amd as m
    m.load_library()
    return m


def _aux(T, E, k, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    return dict(topk_idx=torch.empty((T, k), **i32),
                topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
                counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                dropped=torch.empty(T * k, dtype=torch.uint8, device=dev))


def _same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def _compare(moe, d, T, k, cf, label):
    """One noalloc call on the first T tokens against moe_layer_forward."""
    x = d["x"][:T].contiguous()
    E = d["wg"].shape[0]
    H = x.shape[1]
    ref, rax = moe.moe_layer_forward(x, d["wr"], d["wg"], d["wu"], d["wd"], k=k,
                                     capacity_factor=cf, s_gate=d["sg"], s_up=d["su"],
                                     s_down=d["sd"], aux=True)
    out = torch.full((T, H), 7.0, dtype=x.dtype, device=x.device)
    ax = _aux(T, E, k, x.device)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    moe.moe_layer_forward_noalloc(x, d["wr"], d["wg"], d["wu"], d["wd"], k=k,
                                  capacity_factor=cf, s_gate=d["sg"], s_up=d["su"],
                                  s_down=d["sd"], out=out, aux=ax)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    log(f"noalloc {label}: T={T} H={H} E={E} k={k} cf={cf}")
    assert _same(out, ref), f"{label}: out differs from moe_layer_forward"
    for n in ("topk_idx", "topk_w", "counts", "offsets", "dropped"):
        assert _same(ax[n], rax[n]), f"{label}: {n} differs"
    return out


CASES = [
    # (config, first T, second T, capacity factor)
    (synth.get_config("p_bf16_dec").with_(T=16), 16, 5, None),
    (synth.get_config("p_i8_dec").with_(T=12), 12, 3, 1.0),
    (synth.get_config("p_i4_dec"), 9, 1, None),
    (synth.get_config("tiny"), 32, 7, 1.25),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_noalloc_equals_layer_forward(moe, case):
    cfg, t1, t2, cf = case
    d = to_device(synth.generate_host(cfg))
    a = _compare(moe, d, t1, cfg.k, cf, cfg.name + " (first)")
    b = _compare(moe, d, t2, cfg.k, cf, cfg.name + " (second, smaller)")
    assert a.shape[0] == t1 and b.shape[0] == t2


def test_noalloc_grok1_decode_shape(moe):
    # the Grok-1 decode shape (H = 6144, F = 32768, bf16): 8 tokens, then 2
    cfg = synth.CONFIGS["decode"]
    dv = generate_device(cfg, "cuda")
    d = dict(x=dv.x, wr=dv.wr, wg=dv.wg, wu=dv.wu, wd=dv.wd, sg=None, su=None, sd=None)
    _compare(moe, d, 8, 2, None, "grok1 decode (first)")
    _compare(moe, d, 2, 2, None, "grok1 decode (second, smaller)")
    # 17 tokens take the tiled path, whose workspace exceeds the scratch
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_noalloc(torch.empty((17, cfg.H), dtype=torch.bfloat16,
                                                  device="cuda"), d["wr"], d["wg"], d["wu"],
                                      d["wd"])
    assert ei.value.status == 2
    del dv, d
    torch.cuda.empty_cache()
