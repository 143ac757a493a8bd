"""Expert capacity with drops (the Go chapter, "What was simplified": an
expert accepts a bounded number of tokens and the overflow is dropped),
through the C ABI against the oracle.  The oracle's reading: an expert keeps
its first C assignments in flat order t*k + j, a dropped slot adds nothing,
the kept gates are not renormalised, and counts / Importance stay the
router's view of every assignment."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_common import check_outputs, check_routing, require_gpu, run_forward
from helpers import BF16, F32, GELU, SWIGLU, random_layer
from sparse_mixture_experts_07_amd import binding as B
from sparse_mixture_experts_07_amd.device import DeviceLayer

pytestmark = pytest.mark.gpu

# (layer, capacity factor); T*k <= 4096 runs the one-workgroup grouping
# kernel, larger batches the multi-workgroup one.
CASES = {
    "fused-swiglu-bf16": (dict(T=300, d=128, h=256, E=6, k=2, act=SWIGLU, dtype=BF16, bias=True), 0.75),
    "fused-gelu-bias-f32": (dict(T=200, d=64, h=128, E=5, k=2, act=GELU, dtype=F32, expert_bias=True, bias=True), 1.0),
    "fused-shared-bf16": (dict(T=257, d=128, h=192, E=9, k=3, act=SWIGLU, dtype=BF16, S=1, bias=True), 0.5),
    "fused-e64-bf16": (dict(T=500, d=64, h=64, E=64, k=6, act=SWIGLU, dtype=BF16, bias=True), 1.0),
    "multi-swiglu-bf16": (dict(T=3000, d=64, h=64, E=16, k=2, act=SWIGLU, dtype=BF16, bias=True), 1.0),
    "multi-gelu-f32": (dict(T=2500, d=64, h=128, E=8, k=2, act=GELU, dtype=F32, bias=True), 1.1),
    "multi-shared-bf16": (dict(T=2100, d=128, h=128, E=12, k=3, act=SWIGLU, dtype=BF16, S=1, bias=True), 0.6),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _capacity(c, factor):
    cap = B.moe_expert_capacity(c["T"], c["k"], c["E"], factor)
    assert cap == oracle.expert_capacity(c["T"], c["k"], c["E"], factor)
    return cap


@pytest.mark.parametrize("name", list(CASES))
def test_forward_with_capacity_every_token(name):
    """Routing and counts bit-exact (router view), Importance and the load
    statistics over every assignment, every output row against the oracle
    with the same drops."""
    kw, factor = CASES[name]
    L = random_layer(11, **kw)
    cap = _capacity(kw, factor)
    res, _, _ = run_forward(L, capacity=cap)
    ridx, rw = check_routing(L, res["idx"], res["w"], res["counts"])
    keep = oracle.capacity_keep(L.cfg, ridx, cap)
    assert keep.sum() < keep.size, "the case is meant to drop assignments"
    rc, rimp = oracle.counts(L.cfg, ridx, rw)
    np.testing.assert_allclose(res["importance"], rimp, rtol=1e-5)
    np.testing.assert_allclose(res["stats"], oracle.load_stats(rc, rimp),
                               rtol=1e-4, atol=1e-9)
    check_outputs(L, res["y"], range(L.cfg.T), keep=keep)


@pytest.mark.parametrize("name", ["fused-shared-bf16", "multi-swiglu-bf16", "multi-gelu-f32"])
def test_grouping_with_capacity_bit_exact(name):
    """moe_permute on the oracle's routing: kept group offsets, sources and
    positions (-1 for a dropped slot) bit-exact, x_perm over the kept rows a
    bit-exact gather of x."""
    kw, factor = CASES[name]
    L = random_layer(12, **kw)
    cap = _capacity(kw, factor)
    cfg = L.cfg
    T, k, E, d = cfg.T, cfg.k, cfg.E, cfg.d
    ridx, rw, _ = oracle.route(L)
    keep = oracle.capacity_keep(cfg, ridx, cap)
    roff, rsrc, rpos = oracle.permute_keep(cfg, ridx, keep)
    dl = DeviceLayer.upload(L, capacity=cap)
    dev = dl.x.device
    ws = torch.empty(B.moe_workspace_bytes(dl.cfg), dtype=torch.uint8, device=dev)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    perm_src = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    pos = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    imp = torch.empty(E, dtype=torch.float32, device=dev)
    x_perm = torch.zeros((T * k, d), dtype=dl.x.dtype, device=dev)
    gidx = torch.from_numpy(ridx).to(dev)
    gw = torch.from_numpy(rw.astype(np.float32)).to(dev)
    B.moe_permute(dl.cfg, gidx, gw, dl.x, offsets, perm_src, pos, imp, None, x_perm, ws)
    torch.cuda.synchronize()
    n_kept = int(roff[-1])
    assert n_kept < T * k
    assert np.array_equal(offsets.cpu().numpy(), roff)
    assert np.array_equal(perm_src.cpu().numpy()[:n_kept], rsrc)
    assert np.array_equal(pos.cpu().numpy(), rpos)
    # rows past the kept ones are not written
    assert perm_src[n_kept:].eq(-7).all() and x_perm[n_kept:].view(torch.int16).eq(0).all()
    xp = x_perm.view(torch.int16 if cfg.dtype == BF16 else torch.int32).cpu().numpy()
    assert np.array_equal(xp[:n_kept].view(L.x.dtype), L.x[rsrc])
    _, rimp = oracle.counts(cfg, ridx, rw)
    np.testing.assert_allclose(imp.cpu().numpy(), rimp, rtol=1e-5)


@pytest.mark.parametrize("T", [300, 2500])
def test_large_capacity_equals_no_capacity(T):
    """A capacity at or above the largest group drops nothing: bitwise the
    output without a capacity."""
    L = random_layer(13, T=T, d=64, h=128, E=8, k=2, act=SWIGLU, dtype=BF16, bias=True)
    ref, _, _ = run_forward(L)
    cap = int(ref["counts"].max())
    got, _, _ = run_forward(L, capacity=cap)
    assert np.array_equal(got["y"], ref["y"])
    for key in ("idx", "w", "counts", "importance", "stats"):
        assert np.array_equal(got[key], ref[key]), key
    less, _, _ = run_forward(L, capacity=cap - 1)
    assert not np.array_equal(less["y"], ref["y"])


@pytest.mark.parametrize("S", [0, 1])
def test_tokens_with_every_slot_dropped(S):
    """A bias sends every token to experts 0 and 1 first; with capacity 5
    only the first five tokens keep their slots.  The other rows are exactly
    zero (no shared expert) or exactly the shared expert's output."""
    L = random_layer(14, T=64, d=64, h=128, E=8, k=2, act=SWIGLU, dtype=BF16, S=S)
    L.b_gate = np.zeros(8, np.float32)
    L.b_gate[:2] = 1e4
    res, _, _ = run_forward(L, capacity=5)
    ridx, _ = check_routing(L, res["idx"], res["w"], res["counts"])
    assert np.all(np.sort(ridx, axis=1) == [0, 1])
    keep = oracle.capacity_keep(L.cfg, ridx, 5)
    assert keep.reshape(64, 2)[:5].all() and not keep.reshape(64, 2)[5:].any()
    check_outputs(L, res["y"], range(64), keep=keep)
    if S == 0:
        assert np.all(res["y"][5:] == 0.0)
    else:
        assert np.all(np.abs(res["y"][5:]).max(axis=1) > 0)
