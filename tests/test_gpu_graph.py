"""The calls only enqueue work on the caller's stream, so a whole layer can
be captured in a HIP graph: moe_forward (and the training step's
moe_backward) captured once, replayed several times with other eager work
and synchronisations between the replays, every replay bitwise equal to the
eager result (outputs overwritten before each replay)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import require_gpu
from helpers import BF16, GELU, SWIGLU, random_layer
from sparse_mixture_experts_07_amd import binding as B
from sparse_mixture_experts_07_amd.device import DeviceLayer, Forward, to_device
from synthetic import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


CASES = {
    "e8-shared-large-groups": (dict(T=600, d=128, h=256, E=8, k=2, act=SWIGLU, dtype=BF16, S=1,
                                    bias=True), 0, 0),
    "e64-multi-segment": (dict(T=3000, d=64, h=64, E=64, k=6, act=SWIGLU, dtype=BF16), 0, 0),
    "e256-router": (dict(T=300, d=64, h=64, E=256, k=8, act=SWIGLU, dtype=BF16, bias=True), 0, 0),
    "gelu-capacity-next-choice": (dict(T=1500, d=64, h=128, E=16, k=2, act=GELU, dtype=BF16,
                                       bias=True, expert_bias=True), 150,
                                  B.MOE_OVERFLOW_NEXT_CHOICE),
}


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else
                  (torch.int64 if t.dtype == torch.float64 else torch.int32)).clone()


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replays(name):
    kw, cap, ov = CASES[name]
    L = random_layer(70, **kw)
    dl = DeviceLayer.upload(L, capacity=cap, overflow=ov)
    fw = Forward(dl)
    outs = lambda: [fw.y, fw.topk_idx, fw.topk_w, fw.counts, fw.importance, fw.stats]
    fw()
    torch.cuda.synchronize()
    ref = [_bits(t) for t in outs()]
    # other eager work between replays: a second layer's forward
    other = Forward(DeviceLayer.upload(random_layer(71, **kw)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the launch-time caches off the capture
        fw()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fw()
    for rep in range(4):
        for t in outs():
            t.view(torch.uint8).fill_(0x5A)
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(outs()):
            assert torch.equal(_bits(t), ref[i]), f"replay {rep}: output {i} differs"


def test_training_step_graph_replays():
    """Forward stages with the training up projection, then moe_backward
    with the Importance loss, captured together."""
    L = random_layer(72, wstd=0.15, T=700, d=128, h=256, E=8, k=2, act=SWIGLU, dtype=BF16,
                     bias=True, S=1)
    dl = DeviceLayer.upload(L)
    c, dev = dl.cfg, dl.x.device
    cfg = L.cfg
    T, k, E, d, h = cfg.T, cfg.k, cfg.E, cfg.d, cfg.h
    R = B.moe_grouped_rows(c)
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    b16 = dict(dtype=torch.bfloat16, device=dev)
    idx, w = torch.empty((T, k), **i32), torch.empty((T, k), **f32)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm_src, pos, imp = torch.empty(T * k, **i32), torch.empty(T * k, **i32), torch.empty(E, **f32)
    x_perm = torch.empty((T * k, d), **b16)
    hidden, preact = torch.empty((R, h), **b16), torch.empty((R, 2 * h), **b16)
    y_perm, y = torch.empty((R, d), **b16), torch.empty((T, d), **b16)
    ws = torch.empty(B.moe_workspace_bytes(c), dtype=torch.uint8, device=dev)
    g_t = dict(dx=torch.empty((T, d), **b16), w_gate=torch.empty((E, d), **f32),
               w_up=torch.empty((E, 2 * h, d), **b16), w_down=torch.empty((E, d, h), **b16),
               b_gate=torch.empty(E, **f32), w_up_shared=torch.empty((1, 2 * h, d), **b16),
               w_down_shared=torch.empty((1, d, h), **b16))
    mg = B.grads(g_t["dx"], g_t["w_gate"], g_t["w_up"], g_t["w_down"], g_t["b_gate"],
                 dw_up_shared=g_t["w_up_shared"], dw_down_shared=g_t["w_down_shared"])
    ws_b = torch.empty(B.moe_backward_workspace_bytes(c), dtype=torch.uint8, device=dev)
    dy = to_device(f32_to_bf16_bits(np.random.default_rng(73).standard_normal(
        (T, d)).astype(np.float32)), dev)
    W = dl.weights()

    def step():
        B.moe_route(c, dl.x, dl.w_gate, dl.b_gate, idx, w, counts)
        B.moe_permute(c, idx, w, dl.x, offsets, perm_src, pos, imp, None, x_perm, ws)
        B.moe_expert_up_train(c, W, x_perm, dl.x, offsets, hidden, preact)
        B.moe_expert_down(c, W, hidden, offsets, y_perm)
        B.moe_combine(c, y_perm, pos, w, y)
        B.moe_backward(c, W, dl.x, dy, idx, w, offsets, pos, x_perm, y_perm, imp, 0.3, mg,
                       ws_b, hidden=hidden, preact=preact)

    outs = [y] + list(g_t.values())
    step()
    torch.cuda.synchronize()
    ref = [_bits(t) for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.view(torch.uint8).fill_(0x3C)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(outs):
            assert torch.equal(_bits(t), ref[i]), f"replay {rep}: output {i} differs"
