"""C-ABI checks that need no GPU: libmoe.so loads, exports every function that
include/moe.h declares, and rejects bad arguments before any HIP call."""
import ctypes as C
import math
import os
import re

import pytest

from sparse_moe_transformer_top_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INV, UNS, WS, HIP = 0, 1, 2, 3, 4
F32, BF16, I8, I4 = 0, 1, 2, 3
P = 0x10000           # fake, 16-byte aligned device address: never dereferenced
MIS = 0x10008         # misaligned fake address


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings(lib):
    assert [lib.moe_status_string(i).decode() for i in range(5)] == [
        "MOE_OK", "MOE_ERR_INVALID_ARGUMENT", "MOE_ERR_UNSUPPORTED",
        "MOE_ERR_WORKSPACE_TOO_SMALL", "MOE_ERR_HIP"]


def router(lib, x=P, xdt=BF16, wr=P, T=8, H=128, E=8, k=2, idx=P, w=P):
    return lib.moe_router_topk(x, xdt, wr, T, H, E, k, idx, w, None, None)


def test_router_argument_errors(lib):
    assert router(lib, x=None) == INV
    assert router(lib, idx=None) == INV
    assert router(lib, T=-1) == INV
    assert router(lib, k=0) == INV
    assert router(lib, k=9) == INV          # k > E
    assert router(lib, E=17, k=2) == UNS
    assert router(lib, k=5, E=8) == UNS
    assert router(lib, H=100) == UNS
    assert router(lib, H=0) == INV
    assert router(lib, xdt=I8) == UNS
    assert router(lib, x=MIS) == INV
    assert "aligned" in lib.moe_last_error().decode()
    assert router(lib, T=2 ** 31) == UNS     # T*k overflows int32 rows
    assert router(lib, T=0) == OK            # empty input: nothing launched


def dispatch(lib, idx=P, T=8, E=8, k=2, cf=0.0, ws=P, nws=None, outs=(P, P, P, P, P)):
    nws = lib.moe_dispatch_workspace_bytes(T, E, k) if nws is None else nws
    return lib.moe_dispatch(idx, T, E, k, cf, *outs, ws, nws, None)


def test_dispatch_argument_errors(lib):
    assert dispatch(lib, idx=None) == INV
    assert dispatch(lib, outs=(P, P, None, P, P)) == INV
    assert dispatch(lib, cf=math.nan) == INV
    assert dispatch(lib, nws=0) == WS
    assert dispatch(lib, ws=None) == WS
    assert dispatch(lib, k=3, E=2) == INV
    assert lib.moe_dispatch_workspace_bytes(5000, 8, 2) >= 5 * 8 * 4


def ffn(lib, act=BF16, wdt=BF16, T=32, H=128, F=256, E=8, k=2, scales=(None, None, None),
        ptrs=None, ws=None, nws=0):
    p = dict(x=P, perm=P, off=P, wg=P, wu=P, wd=P, h=P, y=P)
    p.update(ptrs or {})
    return lib.moe_expert_ffn(p["x"], act, p["perm"], p["off"], T, H, F, E, k, p["wg"], p["wu"],
                              p["wd"], wdt, *scales, p["h"], p["y"], ws, nws, None)


def test_expert_ffn_argument_errors(lib):
    assert ffn(lib, ptrs=dict(h=None)) == INV
    assert ffn(lib, wdt=I8) == INV                          # int8 without scales
    assert ffn(lib, scales=(P, P, P)) == INV                # scales with bf16 weights
    assert ffn(lib, act=F32, wdt=BF16) == UNS
    assert ffn(lib, act=F32, wdt=I8, scales=(P, P, P)) == UNS
    assert ffn(lib, act=I8, wdt=I8, scales=(P, P, P)) == UNS
    assert ffn(lib, F=100) == UNS
    assert ffn(lib, ptrs=dict(wd=MIS)) == INV
    assert ffn(lib, T=0) == OK
    # int4: decode sizes only, H and F multiples of 128, scales required
    assert ffn(lib, wdt=I4, T=16) == INV                    # int4 without scales
    assert ffn(lib, wdt=I4, T=17, scales=(P, P, P)) == UNS
    assert ffn(lib, wdt=I4, T=8, H=192, scales=(P, P, P)) == UNS
    assert ffn(lib, wdt=I4, T=8, F=320, scales=(P, P, P)) == UNS
    assert ffn(lib, act=F32, wdt=I4, T=8, scales=(P, P, P)) == UNS
    # one expert's int4 codes must stay under 2 GiB (32-bit offsets in the kernels)
    assert ffn(lib, wdt=I4, T=8, H=65536, F=65536, scales=(P, P, P)) == UNS
    assert ffn(lib, wdt=I4, T=0, H=65536, F=65536, scales=(P, P, P)) == UNS


def test_stage_entry_points_argument_errors(lib):
    gu = lambda **kw: lib.moe_expert_gate_up(
        kw.get("x", P), BF16, P, P, 32, 128, 256, 8, 2, P, P, kw.get("wdt", BF16),
        kw.get("sg"), kw.get("su"), kw.get("h", P), None)
    assert gu(h=None) == INV
    assert gu(wdt=I8) == INV
    assert gu(wdt=I8, sg=P) == INV
    assert gu(x=MIS) == INV
    dn = lambda **kw: lib.moe_expert_down(
        kw.get("h", P), BF16, P, 32, 128, kw.get("F", 256), 8, 2, P, kw.get("wdt", BF16),
        kw.get("sd"), P, None, 0, None)
    assert dn(h=None) == INV
    assert dn(wdt=I8) == INV
    assert dn(sd=P) == INV
    assert dn(F=200) == UNS


def test_routing_stats_argument_errors(lib):
    st = lib.moe_routing_stats
    assert st(P, P, 8, 8, 2, None, None, None, None) == OK          # nothing requested
    assert st(None, P, 0, 8, 2, None, P, P, None) == OK             # T = 0: nothing per token
    assert st(P, None, 8, 8, 2, P, None, None, None) == INV         # utilisation needs counts
    assert st(None, P, 8, 8, 2, None, P, None, None) == INV         # margin needs logits
    assert st(P, P, 8, 8, 0, None, P, None, None) == INV
    assert st(P, P, 8, 8, 9, None, P, None, None) == INV
    assert st(P, P, 8, 17, 2, None, P, None, None) == UNS
    assert st(P, P, 8, 8, 5, None, P, None, None) == UNS
    assert st(P, P, -1, 8, 2, None, P, None, None) == INV


def test_ep_argument_errors(lib):
    pk = lambda **kw: lib.moe_ep_pack(kw.get("x", P), BF16, P, P, kw.get("T", 8), 128,
                                      kw.get("E", 8), 2, kw.get("R", 2), kw.get("send", P),
                                      kw.get("cnt", P), None)
    assert pk(R=3) == INV                 # E not a multiple of R
    assert pk(R=65, E=8) == UNS
    assert pk(cnt=None) == INV
    assert pk(send=None) == INV
    assert pk(x=MIS) == INV
    rl = lambda **kw: lib.moe_ep_recv_layout(P, kw.get("R", 2), kw.get("El", 4),
                                             kw.get("mr", 100), kw.get("off", P),
                                             kw.get("idx", P), None)
    assert rl(R=0) == UNS
    assert rl(El=17) == UNS
    assert rl(mr=-1) == INV
    assert rl(idx=None) == INV
    assert rl(off=None) == INV
    up = lambda **kw: lib.moe_ep_unpack(kw.get("y", P), BF16, P, P, kw.get("El", 4), 128,
                                        kw.get("mr", 100), kw.get("back", P), None)
    assert up(mr=0) == OK
    assert up(back=None) == INV
    assert up(y=MIS) == INV
    assert up(El=0) == UNS


def test_combine_argument_errors(lib):
    assert lib.moe_combine(None, P, P, 8, 128, 2, BF16, P, None) == INV
    assert lib.moe_combine(P, P, P, 8, 128, 0, BF16, P, None) == INV
    assert lib.moe_combine(P, P, P, 8, 96, 2, BF16, P, None) == UNS
    assert lib.moe_combine(P, P, P, 8, 128, 2, I8, P, None) == UNS
    assert lib.moe_combine(P, P, P, 0, 128, 2, BF16, P, None) == OK


def layer(lib, T=32, H=128, F=256, E=8, k=2, act=BF16, wdt=BF16, cf=0.0, ws=P, nws=None,
          scales=(None, None, None), out=P):
    nws = lib.moe_layer_workspace_bytes(T, H, F, E, k, act, wdt) if nws is None else nws
    return lib.moe_layer_forward(P, act, P, P, P, P, wdt, *scales, T, H, F, E, k, cf, out,
                                 None, None, None, None, None, ws, nws, None)


def test_layer_argument_errors(lib):
    assert layer(lib, out=None) == INV
    assert layer(lib, nws=16) == WS
    assert layer(lib, ws=None) == WS
    assert layer(lib, ws=MIS) == WS
    assert layer(lib, cf=math.nan) == INV
    assert layer(lib, act=F32, wdt=I8, scales=(P, P, P)) == UNS
    assert layer(lib, k=3, E=2) == INV


def layer_noalloc(lib, T=16, H=6144, F=32768, E=8, k=2, act=BF16, wdt=BF16, cf=0.0,
                  scales=(None, None, None), out=P, x=P):
    return lib.moe_layer_forward_noalloc(x, act, P, P, P, P, wdt, *scales, T, H, F, E, k, cf, out,
                                         None, None, None, None, None, None)


def test_layer_noalloc_argument_errors(lib):
    # every check runs before the scratch lookup and any launch
    assert layer_noalloc(lib, out=None) == INV
    assert layer_noalloc(lib, x=MIS) == INV
    assert layer_noalloc(lib, cf=math.nan) == INV
    assert layer_noalloc(lib, act=F32, wdt=I8, scales=(P, P, P)) == UNS
    # a workspace above the fixed scratch: rejected, nothing enqueued
    n = lib.moe_layer_workspace_bytes(17, 6144, 32768, 8, 2, BF16, BF16)
    assert n > _lib.NOALLOC_SCRATCH_BYTES
    assert layer_noalloc(lib, T=17) == UNS
    assert "workspace" in lib.moe_last_error().decode()
    # the Grok-1 decode sizes fit the scratch
    for T in (1, 8, 16):
        for wdt, sc in ((BF16, (None, None, None)), (I8, (P, P, P)), (I4, (P, P, P))):
            assert lib.moe_layer_workspace_bytes(T, 6144, 32768, 8, 2, BF16, wdt) <= \
                _lib.NOALLOC_SCRATCH_BYTES
    assert layer_noalloc(lib, T=0) == OK      # empty input with no optional outputs: no launch


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_workspace_sizes(lib):
    T, H, F, E, k = 8192, 6144, 32768, 8, 2
    n = lib.moe_layer_workspace_bytes(T, H, F, E, k, BF16, BF16)
    # h [T*k, F] and y_perm [T*k, H] in bf16 dominate; plus 192 MiB of
    # float32 partials for the down projection's split tail tiles
    assert n >= T * k * (F + H) * 2 + (192 << 20)
    assert n < T * k * (F + H) * 2 + (256 << 20)
    assert lib.moe_expert_ffn_workspace_bytes(T, H, F, E, k, BF16, BF16) == 192 << 20
    assert lib.moe_layer_workspace_bytes(T, H, F, E, k, F32, F32) > n
    assert lib.moe_layer_workspace_bytes(0, H, F, E, k, BF16, BF16) > 0
    assert lib.moe_expert_ffn_workspace_bytes(T, H, F, E, k, BF16, BF16) >= 0


def fwd_train(lib, T=32, H=128, F=256, E=8, k=2, act=BF16, wdt=BF16, cf=0.0, res=P, nres=None,
              out=P, x=P):
    nres = lib.moe_layer_train_reserve_bytes(T, H, F, E, k) if nres is None else nres
    return lib.moe_layer_forward_train(x, act, P, P, P, P, wdt, T, H, F, E, k, cf, out, res, nres,
                                       None)


def bwd(lib, T=32, H=128, F=256, E=8, k=2, act=BF16, wdt=BF16, res=P, nres=None, ws=P, nws=None,
        dx=P, dwr=P, dout=P):
    nres = lib.moe_layer_train_reserve_bytes(T, H, F, E, k) if nres is None else nres
    nws = lib.moe_layer_backward_workspace_bytes(T, H, F, E, k) if nws is None else nws
    return lib.moe_layer_backward(P, act, P, P, P, P, wdt, T, H, F, E, k, dout, res, nres, dx, dwr,
                                  P, P, P, ws, nws, None)


def test_training_argument_errors(lib):
    assert fwd_train(lib, out=None) == INV
    assert fwd_train(lib, x=MIS) == INV
    assert fwd_train(lib, nres=64) == WS
    assert fwd_train(lib, res=None) == WS
    assert fwd_train(lib, res=MIS) == WS
    assert fwd_train(lib, cf=math.nan) == INV
    assert fwd_train(lib, act=F32, wdt=F32) == UNS       # bf16 only
    assert fwd_train(lib, wdt=I8) == UNS
    assert fwd_train(lib, H=96) == UNS
    assert fwd_train(lib, T=2 ** 30 - 16, k=2) == UNS     # T*k + 64 slack rows reach 2^31
    assert bwd(lib, dx=None) == INV
    assert bwd(lib, dout=MIS) == INV
    assert bwd(lib, dwr=None) == INV
    assert bwd(lib, nres=64) == WS
    assert bwd(lib, nws=64) == WS
    assert bwd(lib, ws=None) == WS
    assert bwd(lib, act=F32, wdt=F32) == UNS
    assert bwd(lib, k=5, E=8) == UNS
    assert bwd(lib, E=17) == UNS


def test_training_sizes(lib):
    T, H, F, E, k = 8192, 6144, 32768, 8, 2
    N = T * k
    r = lib.moe_layer_train_reserve_bytes(T, H, F, E, k)
    # g, u, h [N, F] and y_perm [N, H] in bf16 dominate the reserve
    assert N * (3 * F + H) * 2 + (192 << 20) <= r < N * (3 * F + H) * 2 + (208 << 20)
    w = lib.moe_layer_backward_workspace_bytes(T, H, F, E, k)
    # dy, [dg | du] and the gathered x rows (64 slack rows each), dh and the
    # per-row dx, all bf16, and 192 MiB of float32 partial tiles; no
    # transposed weights
    rows = (N + 64) * (H + 2 * F + H) * 2 + N * (F + H) * 2 + (192 << 20)
    assert rows <= w < rows + 64 * 2 ** 20
    assert lib.moe_layer_train_reserve_bytes(0, H, F, E, k) > 0
    assert lib.moe_layer_backward_workspace_bytes(-1, H, F, E, k) == 0


def test_backward_step_argument_errors(lib):
    T, H, F, E, k = 32, 128, 256, 8, 2
    nres = lib.moe_layer_train_reserve_bytes(T, H, F, E, k)
    nws = lib.moe_layer_backward_workspace_bytes(T, H, F, E, k)
    data = lambda **kw: lib.moe_layer_backward_data(
        P, kw.get("act", BF16), P, P, P, P, BF16, T, H, F, E, k, kw.get("dout", P), P, nres,
        kw.get("dx", P), kw.get("dwr", P), kw.get("ws", P), kw.get("nws", nws), None)
    wts = lambda **kw: lib.moe_layer_backward_weights(
        kw.get("T", T), H, F, E, k, P, kw.get("nres", nres), kw.get("dwg", P), P, P,
        kw.get("ws", P), nws, None)
    assert data(dx=None) == INV
    assert data(dwr=MIS) == INV
    assert data(act=F32) == UNS
    assert data(nws=nws - 1) == WS
    assert wts(dwg=None) == INV
    assert wts(dwg=MIS) == INV
    assert wts(ws=None) == WS
    assert wts(nres=16) == WS
    assert wts(T=-1) == INV
    # the fused call checks the weight step's pointers before enqueuing anything
    assert lib.moe_layer_backward(P, BF16, P, P, P, P, BF16, T, H, F, E, k, P, P, nres, P, P, MIS,
                                  P, P, P, nws, None) == INV
