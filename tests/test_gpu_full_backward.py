"""The training step at the benchmarked sizes, in the launch configuration
`bench.py --backward` times (the training up projection keeps the
pre-activations; the Importance loss weight 0.01).  GPT-2 shape: every
gradient against the float64 autograd oracle.  Mixtral and DeepSeek-V3
shapes, too large for the whole graph on the CPU: dx rows of a token
sample, and the weight gradients of sampled hidden units of the largest,
the smallest and (DeepSeek-V3) the shared expert, against the oracle's
slices of the same gradient (pinned to the whole graph on small layers).
The same with the noisy gate (its smooth-Load loss weight 0.01, as
`bench.py --noisy --backward`), plus output rows.  The router's weight
gradients (W_g, b_g, and W_noise with the noisy gate) at those two shapes
against the oracle's router slice: every slot's float64 expert output held
fixed (pinned to the whole graph on small layers), which takes one full
oracle forward of the batch on the CPU."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_common import max_rel, require_gpu, sample_tokens, to_f64
from sparse_mixture_experts_07_amd import binding as B
from sparse_mixture_experts_07_amd.device import DeviceLayer, to_device
from synthetic import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

GRAD_TOL = 2e-2
IMP_W = 0.01
LOAD_W = 0.01


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def training_step(L, dy_bits, noise=None):
    """Stage calls of the training step (moe_route .. moe_combine with the
    training up projection, then moe_backward; noise: the noisy gate with
    these draws and the layer's w_noise, the smooth-Load loss weight
    LOAD_W); the gradients and y on the host as float64, and the routing."""
    cfg = L.cfg
    dl = DeviceLayer.upload(L)
    c, dev = dl.cfg, dl.x.device
    T, k, E, d, h, S = cfg.T, cfg.k, cfg.E, cfg.d, cfg.h, cfg.S
    nup = cfg.n_up
    R = B.moe_grouped_rows(c)
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    b16 = dict(dtype=torch.bfloat16, device=dev)
    idx, w = torch.empty((T, k), **i32), torch.empty((T, k), **f32)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm_src, pos = torch.empty(T * k, **i32), torch.empty(T * k, **i32)
    imp = torch.empty(E, **f32)
    x_perm = torch.empty((T * k, d), **b16)
    hidden, preact = torch.empty((R, h), **b16), torch.empty((R, nup), **b16)
    y_perm, y = torch.empty((R, d), **b16), torch.empty((T, d), **b16)
    ws = torch.empty(B.moe_workspace_bytes(c), dtype=torch.uint8, device=dev)
    W = dl.weights()
    nz = None
    if noise is None:
        B.moe_route(c, dl.x, dl.w_gate, dl.b_gate, idx, w, counts)
    else:
        wn, n_d = to_device(L.w_noise, dev), to_device(noise, dev)
        clean, scale = torch.empty((T, E), **f32), torch.empty((T, E), **f32)
        load, imp_n = torch.empty(E, **f32), torch.empty(E, **f32)
        cv2 = torch.empty(2, dtype=torch.float64, device=dev)
        B.moe_route_noisy(c, dl.x, dl.w_gate, dl.b_gate, wn, n_d, clean, scale, idx, w, counts,
                          imp_n, load, cv2, ws)
        dw_noise = torch.empty((E, d), **f32)
        nz = B.noisy_grad(wn, n_d, clean, scale, dw_noise, load, LOAD_W)
    B.moe_permute(c, idx, w, dl.x, offsets, perm_src, pos, imp, None, x_perm, ws)
    B.moe_expert_up_train(c, W, x_perm, dl.x, offsets, hidden, preact)
    B.moe_expert_down(c, W, hidden, offsets, y_perm)
    B.moe_combine(c, y_perm, pos, w, y)
    del ws
    g = dict(dx=torch.empty((T, d), **b16), w_gate=torch.empty((E, d), **f32),
             w_up=torch.empty((E, nup, d), **b16), w_down=torch.empty((E, d, h), **b16),
             b_gate=torch.empty(E, **f32) if L.b_gate is not None else None,
             w_up_shared=torch.empty((1, nup, d), **b16) if S else None,
             w_down_shared=torch.empty((1, d, h), **b16) if S else None)
    mg = B.grads(g["dx"], g["w_gate"], g["w_up"], g["w_down"], g["b_gate"],
                 dw_up_shared=g["w_up_shared"], dw_down_shared=g["w_down_shared"])
    ws_b = torch.empty(B.moe_backward_workspace_bytes(c), dtype=torch.uint8, device=dev)
    B.moe_backward(c, W, dl.x, to_device(dy_bits, dev), idx, w, offsets, pos, x_perm, y_perm,
                   imp, IMP_W, mg, ws_b, hidden=hidden, preact=preact, noisy=nz)
    torch.cuda.synchronize()
    out = {("x" if n == "dx" else n): to_f64(t) for n, t in g.items() if t is not None}
    out["y"] = to_f64(y)
    if noise is not None:
        out["w_noise"] = to_f64(dw_noise)
    ridx = idx.cpu().numpy()
    del dl, ws_b, x_perm, hidden, preact, y_perm, g, mg
    torch.cuda.empty_cache()
    return out, ridx


def _dy(cfg, seed=3):
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(
        (cfg.T, cfg.d)).astype(np.float32))


@pytest.mark.timeout(900)
def test_full_size_training_step_gpt2():
    cfg = synthetic.BY_NAME["gpt2-moe"]
    L = synthetic.make_inputs(cfg)
    dy = _dy(cfg)
    got, idx = training_step(L, dy)
    ridx, _, _ = oracle.route(L)
    assert np.array_equal(idx, ridx)
    ref = oracle.backward.backward(L, bf16_bits_to_f32(dy), importance_weight=IMP_W, idx=ridx)
    errs = {}
    for n, r in ref.items():
        errs[n] = max_rel(got[n].reshape(r.shape), r)
        assert errs[n] <= GRAD_TOL, f"{n}: max-relative error {errs[n]:.3e}"
    print({n: f"{e:.2e}" for n, e in errs.items()})


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name,ntok,noisy,router", [("mixtral-8x7b", 12, False, True),
                                                    ("deepseek-v3", 6, False, True),
                                                    ("mixtral-8x7b", 8, True, True),
                                                    ("deepseek-v3", 4, True, False)])
def test_full_size_training_step_sampled(name, ntok, noisy, router):
    cfg = synthetic.BY_NAME[name]
    L = synthetic.make_inputs(cfg)
    noise = sel = None
    if noisy:
        L.w_noise, noise = synthetic.make_noisy_gate(cfg)
    dy = _dy(cfg)
    got, idx = training_step(L, dy, noise)
    if noisy:
        sel = oracle.backward.noisy_selection(L, noise)
        ridx = sel[0]
    else:
        ridx, _, _ = oracle.route(L)
    assert np.array_equal(idx, ridx)
    dyf = bf16_bits_to_f32(dy)
    errs = {}
    toks = sample_tokens(cfg.T, ntok, seed=1)[:ntok]
    if noisy:   # the output rows with the noisy gate
        r = oracle.route_noisy(L, noise)
        xs = bf16_bits_to_f32(L.x).astype(np.float64)
        yref = np.zeros((len(toks), cfg.d))
        for a, t in enumerate(toks):
            for j in range(cfg.k):
                yref[a] += r["w"][t, j] * oracle.expert(L, int(r["idx"][t, j]), xs[t])
            if cfg.S:
                yref[a] += oracle.expert(L, cfg.E, xs[t])
        errs["y"] = max_rel(got["y"][toks], yref)
    # dx rows: one token at a time (only its experts go to float64)
    ref_dx = np.concatenate([oracle.backward.dx_rows(L, dyf, [t], IMP_W, idx=ridx, noise=noise,
                                                     load_weight=LOAD_W, selection=sel)
                             for t in toks])
    errs["x"] = max_rel(got["x"][toks], ref_dx)
    # hidden units of the largest and the smallest non-empty group (and the
    # shared expert)
    cnt = np.bincount(ridx.ravel(), minlength=cfg.E)
    nz = np.flatnonzero(cnt)
    experts = [int(nz[np.argmax(cnt[nz])]), int(nz[np.argmin(cnt[nz])])]
    if cfg.S:
        experts.append(cfg.E)
    units = np.array([0, 1, cfg.h // 2, cfg.h - 1])
    for e in experts:
        ref = oracle.backward.expert_unit_grads(L, dyf, e, units, idx=ridx, noise=noise,
                                                selection=sel)
        up = got["w_up_shared"][0] if e == cfg.E else got["w_up"][e]
        down = got["w_down_shared"][0] if e == cfg.E else got["w_down"][e]
        gup = np.stack([up[units], up[units + cfg.h]])   # SwiGLU: gate rows, up rows
        errs[f"w_up[{e}]"] = max_rel(gup, ref["w_up"])
        errs[f"w_down[{e}]"] = max_rel(down[:, units], ref["w_down"])
    if router:   # every router weight gradient, from every slot's expert output
        sdy = oracle.backward.slot_dy_products(L, dyf, ridx)
        ref = oracle.backward.router_grads(L, sdy, IMP_W, idx=ridx, noise=noise,
                                           load_weight=LOAD_W, selection=sel)
        for n, r in ref.items():
            errs[n] = max_rel(got[n].reshape(r.shape), r)
    print(name, "noisy" if noisy else "", {n: f"{v:.2e}" for n, v in errs.items()})
    for n, v in errs.items():
        assert v <= GRAD_TOL, f"{n}: max-relative error {v:.3e}"
