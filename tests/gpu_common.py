"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI
and compare with the oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from sparse_mixture_experts_07_amd import binding as B
from sparse_mixture_experts_07_amd.device import DeviceLayer, Forward, bf16_bits

BF16_TOL = 2e-2   # max |y - y_ref| / max |y_ref| for bf16 layers
F32_TOL = 1e-4    # same measure for fp32 layers
W_RTOL = 2e-6     # kept softmax weights: fp32 expf vs the fp64 oracle


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    B.lib()


def to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        b = bf16_bits(t).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def run_forward(layer, capacity: int = 0, overflow: int = 0):
    """moe_forward on the layer; host copies of every output."""
    dl = DeviceLayer.upload(layer, capacity=capacity, overflow=overflow)
    fw = Forward(dl)
    fw()
    torch.cuda.synchronize()
    out = dict(y=to_f64(fw.y), idx=fw.topk_idx.cpu().numpy(),
               w=fw.topk_w.cpu().numpy(), counts=fw.counts.cpu().numpy(),
               importance=fw.importance.cpu().numpy(),
               stats=fw.stats.cpu().numpy())
    return out, dl, fw


def max_rel(y, ref) -> float:
    den = np.abs(ref).max()
    return float(np.abs(y - ref).max() / (den if den > 0 else 1.0))


def check_routing(layer, idx, w, counts, t0=0):
    ridx, rw, _ = oracle.route(layer, t0=t0, nt=idx.shape[0])
    bad = np.nonzero((idx != ridx).any(1))[0]
    assert bad.size == 0, f"routing differs on tokens {bad[:10] + t0}"
    np.testing.assert_allclose(w, rw, rtol=W_RTOL, atol=1e-7)
    if t0 == 0 and idx.shape[0] == layer.cfg.T:
        rc, _ = oracle.counts(layer.cfg, ridx, rw)
        assert np.array_equal(counts, rc)
    return ridx, rw


def check_outputs(layer, y, tokens, tol=None, keep=None, assign=None):
    """keep: the oracle's capacity mask (dropped slots add nothing); assign:
    the oracle's computing expert of every slot (next-choice re-routing)."""
    tokens = np.asarray(tokens, np.int64)
    ref, _, _ = oracle.forward_tokens(layer, tokens, keep=keep, assign=assign)
    got = y[tokens]
    assert np.all(np.isfinite(got))
    tol = tol or (BF16_TOL if layer.cfg.dtype == 1 else F32_TOL)
    err = max_rel(got, ref)
    assert err <= tol, f"max-relative error {err:.3e} > {tol}"
    return err


def sample_tokens(T: int, n: int = 48, seed: int = 0):
    """n distinct tokens (all of them when T <= n): first, second, middle and
    last always, the rest drawn at random; sorted."""
    if T <= n:
        return list(range(T))
    rng = np.random.default_rng(seed)
    base = sorted({0, 1, T // 2, T - 1})[:n]
    rest = np.setdiff1d(np.arange(T), base)
    extra = rng.choice(rest, size=n - len(base), replace=False).tolist()
    return sorted(base + extra)


def covering_tokens(idx: np.ndarray, n: int, seed: int = 0):
    """At least one token of every non-empty expert group of the selection
    idx [T, k] (so every group size class and every group's tiles of the
    grouped GEMM are compared), first, second, middle and last, filled up to
    n tokens at random; sorted."""
    T = idx.shape[0]
    picked = {0, 1, T // 2, T - 1} & set(range(T))
    covered = set(idx[sorted(picked)].ravel().tolist())
    rng = np.random.default_rng(seed)
    for t in rng.permutation(T):
        new = set(idx[t].tolist()) - covered
        if new:
            picked.add(int(t))
            covered |= new
    assert covered == set(idx.ravel().tolist())
    if len(picked) < n:
        rest = np.setdiff1d(np.arange(T), sorted(picked))
        picked |= set(rng.choice(rest, size=min(rest.size, n - len(picked)),
                                 replace=False).tolist())
    return sorted(picked)
