"""Routing variants through the C ABI against the oracle: the bias that
steers the selection only (the Go chapter on DeepSeek-V3's bias balancing,
section 3 and "Pros, cons and real examples") and the softmax over all E
scores read at the kept experts (techfeed summary, "The hardest part: making
the router trainable"; k = 1 is the Switch Transformer gate).  Every router
kernel (one chain per lane for decode batches, LDS-staged chains for large
batches, register tiles for more than 64 experts) in both gate modes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_common import check_outputs, check_routing, require_gpu, run_forward
from helpers import BF16, F32, GELU, SWIGLU, random_layer
from sparse_mixture_experts_07_amd import binding as B
from sparse_mixture_experts_07_amd.device import DeviceLayer

pytestmark = pytest.mark.gpu

SEL = synthetic.GATE_BIAS_SELECTS
ALL = synthetic.GATE_SOFTMAX_ALL

CASES = {
    # router kernel: one chain per lane, few tokens
    "direct-e8-bf16": dict(T=40, d=128, h=128, E=8, k=2, act=SWIGLU, dtype=BF16),
    "direct-e64-bf16": dict(T=100, d=192, h=64, E=64, k=6, act=SWIGLU, dtype=BF16),
    "direct-e6-gelu-f32": dict(T=50, d=64, h=128, E=6, k=2, act=GELU, dtype=F32, expert_bias=True),
    # LDS-staged chains, large batches
    "lane-e16-bf16": dict(T=1500, d=64, h=64, E=16, k=2, act=SWIGLU, dtype=BF16),
    "lane-e32-f32": dict(T=2100, d=64, h=64, E=32, k=4, act=SWIGLU, dtype=F32),
    # register tiles, more than 64 experts
    "tiled-e100-bf16": dict(T=300, d=128, h=64, E=100, k=3, act=SWIGLU, dtype=BF16),
    "tiled-e256-shared-bf16": dict(T=200, d=64, h=64, E=256, k=8, act=SWIGLU, dtype=BF16, S=1),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("gate", [SEL, ALL], ids=["bias-selects", "softmax-all"])
@pytest.mark.parametrize("name", list(CASES))
def test_gate_mode_every_token(name, gate):
    """Indices, counts and (biased) logits bit-exact, kept weights within the
    fp32 exp tolerance, every output row against the oracle."""
    L = random_layer(31, bias=True, gate=gate, **CASES[name])
    res, dl, _ = run_forward(L)
    ridx, rw = check_routing(L, res["idx"], res["w"], res["counts"])
    if gate == ALL:
        assert np.all(res["w"].sum(1) <= 1.0 + 1e-6)
    c, T, E = dl.cfg, L.cfg.T, L.cfg.E
    logits = torch.empty((T, E), dtype=torch.float32, device=dl.x.device)
    idx = torch.empty((T, L.cfg.k), dtype=torch.int32, device=dl.x.device)
    w = torch.empty((T, L.cfg.k), dtype=torch.float32, device=dl.x.device)
    cnt = torch.empty(E, dtype=torch.int32, device=dl.x.device)
    B.moe_route(c, dl.x, dl.w_gate, dl.b_gate, idx, w, cnt, logits)
    torch.cuda.synchronize()
    _, _, rsc = oracle.route(L, want_scores=True)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), rsc.view(np.uint32))
    assert np.array_equal(w.cpu().numpy(), res["w"])
    check_outputs(L, res["y"], range(T))


@pytest.mark.parametrize("name", ["direct-e8-bf16", "lane-e16-bf16", "tiled-e100-bf16"])
def test_bias_selects_without_bias_is_default_gate(name):
    """With no router bias the bias-selects gate is the default gate,
    bitwise, on every router kernel."""
    L = random_layer(32, bias=False, **CASES[name])
    ref, _, _ = run_forward(L)
    L.cfg = L.cfg.with_(gate=SEL)
    got, _, _ = run_forward(L)
    for key in ("idx", "w", "counts", "y"):
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("E", [8, 64, 128])
def test_switch_top1_and_dense_softmax(E):
    """softmax-all with k = 1 (Switch gate: the largest probability) and
    with k = E (the whole softmax, summing to 1)."""
    for k in (1, E):
        L = random_layer(33, T=64, d=64, h=64, E=E, k=k, act=SWIGLU, dtype=BF16,
                         bias=True, gate=ALL)
        res, _, _ = run_forward(L)
        check_routing(L, res["idx"], res["w"], res["counts"])
        if k == E:
            np.testing.assert_allclose(res["w"].sum(1), 1.0, rtol=2e-6)
        check_outputs(L, res["y"], range(64))


def test_gate_mode_with_capacity():
    """Gate modes and the expert capacity compose: the oracle's keep mask
    over the same routing."""
    L = random_layer(34, T=600, d=64, h=128, E=8, k=2, act=SWIGLU, dtype=BF16,
                     bias=True, gate=SEL)
    cap = B.moe_expert_capacity(600, 2, 8, 0.8)
    res, _, _ = run_forward(L, capacity=cap)
    ridx, _ = check_routing(L, res["idx"], res["w"], res["counts"])
    keep = oracle.capacity_keep(L.cfg, ridx, cap)
    assert keep.sum() < keep.size
    check_outputs(L, res["y"], range(600), keep=keep)


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("E,k,d", [(6, 2, 64), (8, 2, 192), (16, 3, 128), (32, 4, 2880),
                                   (64, 6, 320)])
def test_logits_output_leaves_routing_unchanged(E, k, d, dtype):
    """moe_route with and without the logits output (decode-sized batches,
    the one-chain-per-lane kernel): indices, weights and counts bitwise
    equal, and the logits bit-exact against the oracle's scores, for token
    counts around a multiple of 64, every gate mode, with and without the
    router bias."""
    for T in (1, 63, 64, 65, 200):
        for gate in (synthetic.GATE_TOPK_SOFTMAX, SEL, ALL):
            for bias in (False, True):
                if gate == SEL and not bias:
                    continue
                L = random_layer(35 + T + E, T=T, d=d, h=64, E=E, k=k, act=SWIGLU,
                                 dtype=dtype, bias=bias, gate=gate)
                dl = DeviceLayer.upload(L)
                c, dev = dl.cfg, dl.x.device
                out = []
                for with_logits in (False, True):
                    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
                    w = torch.empty((T, k), dtype=torch.float32, device=dev)
                    cnt = torch.empty(E, dtype=torch.int32, device=dev)
                    lg = torch.empty((T, E), dtype=torch.float32, device=dev) if with_logits else None
                    B.moe_route(c, dl.x, dl.w_gate, dl.b_gate, idx, w, cnt, lg)
                    torch.cuda.synchronize()
                    out.append((idx.cpu().numpy(), w.cpu().numpy(), cnt.cpu().numpy(),
                                None if lg is None else lg.cpu().numpy()))
                (i0, w0, c0, _), (i1, w1, c1, lg1) = out
                tag = f"T={T} gate={gate} bias={bias}"
                assert np.array_equal(i0, i1), tag
                assert np.array_equal(w0.view(np.uint32), w1.view(np.uint32)), tag
                assert np.array_equal(c0, c1), tag
                _, _, rsc = oracle.route(L, want_scores=True)
                assert np.array_equal(lg1.view(np.uint32), rsc.view(np.uint32)), tag
                check_routing(L, i1, w1, c1)
