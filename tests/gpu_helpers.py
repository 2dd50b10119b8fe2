"""Shared helpers of the GPU parity tests (moving inputs between numpy, the
oracle's storage form and torch device tensors; tolerance checks)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

# Output tolerances (floating point): bf16 activations compare with
# max|d| <= 2e-2 * max|ref| and ||d||_2 / ||ref||_2 <= 1e-2; float32 with 1e-4
# for both ratios. Routing weights (float32 softmax of float32 logits against
# the float64 softmax of exact logits): absolute 2e-5.
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
W_ATOL = 2e-5


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(a: np.ndarray, kind: str, device="cuda") -> torch.Tensor:
    """Host array in storage form -> device tensor (bf16 from uint16 bits)."""
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_array(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array in storage form (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_device(inp, device="cuda"):
    cfg = inp.cfg
    d = dict(x=dev_tensor(inp.x, cfg.act, device), wr=dev_tensor(inp.wr, "f32", device),
             wg=dev_tensor(inp.wg, cfg.wdt, device), wu=dev_tensor(inp.wu, cfg.wdt, device),
             wd=dev_tensor(inp.wd, cfg.wdt, device))
    for n in ("sg", "su", "sd"):
        v = getattr(inp, n)
        d[n] = None if v is None else dev_tensor(v, "f32", device)
    return d


def out_as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def check_close(got: np.ndarray, ref: np.ndarray, act: str, what: str = ""):
    max_tol, l2_tol = TOL[act]
    d = got.astype(np.float64) - ref
    scale = float(np.abs(ref).max())
    nrm = float(np.linalg.norm(ref))
    max_ratio = float(np.abs(d).max()) / scale if scale > 0 else float(np.abs(d).max())
    l2_ratio = float(np.linalg.norm(d)) / nrm if nrm > 0 else float(np.linalg.norm(d))
    assert max_ratio <= max_tol and l2_ratio <= l2_tol, (
        f"{what}: max|d|/max|ref| = {max_ratio:.3e} (tol {max_tol}), "
        f"||d||/||ref|| = {l2_ratio:.3e} (tol {l2_tol})")
    return max_ratio, l2_ratio


def check_routing(idx_gpu: np.ndarray, w_gpu: np.ndarray, routing: "oracle.Routing"):
    """Indices bit-exact except tie-flagged tokens; weights within W_ATOL.
    Returns the mask of tokens whose indices differ (all tie-flagged)."""
    diff = np.any(idx_gpu != routing.idx, axis=1)
    assert not np.any(diff & ~routing.tie), (
        f"{int(np.sum(diff & ~routing.tie))} non-tie tokens routed differently")
    same = ~diff
    if same.any():
        assert np.max(np.abs(w_gpu[same] - routing.w[same])) <= W_ATOL
    # structural checks that hold for every token
    assert np.all(idx_gpu >= 0) and np.all(idx_gpu < routing.l32.shape[1])
    if idx_gpu.shape[1] > 1:
        assert np.all(np.diff(np.sort(idx_gpu, axis=1), axis=1) > 0)
    assert np.allclose(w_gpu.sum(axis=1), 1.0, atol=1e-6)
    return diff


def check_topk_valid(idx_gpu: np.ndarray, routing: "oracle.Routing", tie_tol: float = 1e-4):
    """Every token's selection is a correct top-k choice: the expert in slot j
    has the j-th largest float64 logit up to the tie tolerance (where near-
    equal logits make several choices correct, any of them passes)."""
    k = idx_gpu.shape[1]
    l64 = routing.l64
    ranked = -np.sort(-l64, axis=1)[:, :k]
    sel = np.take_along_axis(l64, idx_gpu.astype(np.int64), axis=1)
    scale = np.maximum(1.0, np.abs(l64).max(axis=1, keepdims=True))
    bad = np.abs(sel - ranked) > k * tie_tol * scale
    assert not bad.any(), f"{int(bad.any(axis=1).sum())} tokens with an invalid top-k choice"


def gpu_routing(idx_gpu: np.ndarray, w_gpu: np.ndarray, routing: "oracle.Routing"):
    """Checks the GPU's routing against the oracle's (check_routing, then the
    validity of every choice) and returns the indices the reference must use:
    None when they are the oracle's own, else the GPU's (differing only on
    tie-flagged tokens, where both choices are correct)."""
    diff = check_routing(idx_gpu, w_gpu, routing)
    check_topk_valid(idx_gpu, routing)
    if diff.any():
        log(f"  {int(diff.sum())} tie-flagged tokens ordered differently: reference on the "
            "GPU's own choice")
        return idx_gpu
    return None


def check_weights(w_gpu: np.ndarray, routing: "oracle.Routing"):
    assert np.max(np.abs(w_gpu - routing.w)) <= W_ATOL


def check_dispatch_equal(got: dict, ref: "oracle.Dispatch"):
    assert np.array_equal(got["counts"], ref.counts)
    assert np.array_equal(got["offsets"], ref.offsets)
    assert np.array_equal(got["perm"], ref.perm)
    assert np.array_equal(got["slot_row"], ref.slot_row)
    assert np.array_equal(got["dropped"], ref.dropped)


class LazyExperts:
    """Per-expert host copies of a device weight tensor, fetched on access."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, e):
        return host_array(self.t[e])

    def __len__(self):
        return self.t.shape[0]
