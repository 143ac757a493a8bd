"""Pins of the float64 autograd backward in oracle/backward.py (CPU only).

The differentiated function is the layer forward with the oracle's float32
selection held fixed; it is pinned to the C oracle's forward, and its
gradients to finite differences (torch.autograd.gradcheck) and to exact
invariances of the gate."""
import numpy as np
import pytest
import torch

import oracle
from helpers import GELU, SWIGLU, random_layer

B = oracle.backward


def _layer(seed, act, S=0, bias=True, expert_bias=False, T=7, d=6, h=5, E=4, k=2):
    return random_layer(seed, T=T, d=d, h=h, E=E, k=k, act=act, S=S, bias=bias,
                        expert_bias=expert_bias)


@pytest.mark.parametrize("act,S,eb", [(GELU, 0, True), (SWIGLU, 0, False), (SWIGLU, 1, False)])
def test_forward_matches_the_c_oracle(act, S, eb):
    """The float64 torch forward is the C oracle's forward (up to the fp32
    vs fp64 router scores), with and without an expert capacity."""
    L = _layer(1, act, S, expert_bias=eb, T=30, d=16, h=12, E=5, k=2)
    idx, _, _ = oracle.route(L)
    p = B.params(L)
    y, g, imp, _ = B.forward(L, p, idx)
    yc, _, wc = oracle.forward_tokens(L, range(30))
    np.testing.assert_allclose(y.detach().numpy(), yc, rtol=1e-6, atol=1e-7 * np.abs(yc).max())
    np.testing.assert_allclose(g.detach().numpy(), wc, rtol=1e-6)
    _, rimp = oracle.counts(L.cfg, idx, wc)
    np.testing.assert_allclose(imp.detach().numpy(), rimp, rtol=1e-6)
    keep = oracle.capacity_keep(L.cfg, idx, 8)
    assert 0 < keep.sum() < keep.size
    yk, _, _, _ = B.forward(L, p, idx, keep)
    yck, _, _ = oracle.forward_tokens(L, range(30), keep=keep)
    np.testing.assert_allclose(yk.detach().numpy(), yck, rtol=1e-6, atol=1e-7 * np.abs(yck).max())


@pytest.mark.parametrize("act,S,eb,imp_w,cap", [
    (GELU, 0, True, 0.0, 0), (SWIGLU, 0, False, 0.0, 0), (SWIGLU, 1, False, 0.0, 0),
    (SWIGLU, 0, False, 0.7, 0), (GELU, 0, True, 0.3, 3), (SWIGLU, 1, False, 0.5, 4)])
def test_gradients_match_finite_differences(act, S, eb, imp_w, cap):
    """torch.autograd.gradcheck of <dy, y> + w * CV^2(Importance) in every
    input, with the selection fixed (and an expert capacity)."""
    L = _layer(2, act, S, expert_bias=eb)
    idx, _, _ = oracle.route(L)
    keep = oracle.capacity_keep(L.cfg, idx, cap) if cap else None
    if cap:
        assert 0 < keep.sum() < keep.size
    dy = torch.from_numpy(np.random.default_rng(3).standard_normal((L.cfg.T, L.cfg.d)))
    p = B.params(L)
    names = list(p)

    def f(*ts):
        return B.loss(L, dict(zip(names, ts)), idx, dy, keep, imp_w)

    assert torch.autograd.gradcheck(f, tuple(p[n] for n in names), eps=1e-6, atol=1e-6, rtol=1e-5)
    g = B.backward(L, dy.numpy(), keep, imp_w, idx=idx)
    assert set(g) == set(names)


def test_bias_gradient_sums_to_zero_and_top1_router_gets_none():
    """Adding one constant to every router bias changes no kept softmax, so
    the bias gradients sum to 0; with k = 1 the gate is 1 whatever the
    scores, so the router gets no gradient at all."""
    L = _layer(4, SWIGLU, 1, T=20, d=8, h=6, E=6, k=3)
    dy = np.random.default_rng(5).standard_normal((20, 8))
    g = B.backward(L, dy, importance_weight=0.4)
    assert abs(g["b_gate"].sum()) <= 1e-12 * np.abs(g["b_gate"]).sum()
    assert np.abs(g["w_gate"]).max() > 0
    L1 = _layer(6, GELU, 0, expert_bias=True, T=10, d=8, h=6, E=4, k=1)
    g1 = B.backward(L1, np.random.default_rng(7).standard_normal((10, 8)), importance_weight=0.0)
    assert np.all(g1["w_gate"] == 0) and np.all(g1["b_gate"] == 0)


def test_gradients_are_linear_in_dy_and_dropped_slots_get_none():
    """Gradients of <dy, y> are linear in dy; an expert whose every slot is
    dropped by the capacity gets no weight gradient."""
    L = _layer(8, SWIGLU, 0, T=12, d=6, h=4, E=3, k=2)
    rng = np.random.default_rng(9)
    d1, d2 = rng.standard_normal((12, 6)), rng.standard_normal((12, 6))
    g1, g2 = B.backward(L, d1), B.backward(L, d2)
    g12 = B.backward(L, 2.0 * d1 - d2)
    for n in g1:
        np.testing.assert_allclose(g12[n], 2.0 * g1[n] - g2[n], rtol=1e-10, atol=1e-12)
    idx, _, _ = oracle.route(L)
    keep = np.ones(12 * 2, np.uint8)
    keep[(idx == 1).reshape(-1)] = 0
    gk = B.backward(L, d1, keep=keep, idx=idx)
    assert np.all(gk["w_up"][1] == 0) and np.all(gk["w_down"][1] == 0)
    assert np.abs(gk["w_up"][0]).max() > 0


@pytest.mark.parametrize("gate", [1, 2], ids=["bias-selects", "softmax-all"])
def test_gate_modes_forward_and_gradients(gate):
    """The other gate modes: the torch forward equals the C oracle's, and
    gradcheck holds; the bias-selects gate gives the bias no gradient."""
    L = random_layer(9, T=7, d=6, h=5, E=5, k=2, act=SWIGLU, bias=True, gate=gate)
    idx, _, _ = oracle.route(L)
    p = B.params(L)
    y, g, _, _ = B.forward(L, p, idx)
    yc, _, wc = oracle.forward_tokens(L, range(7))
    np.testing.assert_allclose(y.detach().numpy(), yc, rtol=1e-6, atol=1e-7 * np.abs(yc).max())
    np.testing.assert_allclose(g.detach().numpy(), wc, rtol=1e-6)
    dy = torch.from_numpy(np.random.default_rng(10).standard_normal((7, 6)))
    names = list(p)

    def f(*ts):
        return B.loss(L, dict(zip(names, ts)), idx, dy, None, 0.3)

    assert torch.autograd.gradcheck(f, tuple(p[n] for n in names), eps=1e-6, atol=1e-6, rtol=1e-5)
    gr = B.backward(L, dy.numpy(), importance_weight=0.3, idx=idx)
    if gate == 1:
        assert np.all(gr["b_gate"] == 0)
    else:
        assert np.abs(gr["b_gate"]).max() > 0


def test_rerouted_forward_and_gradients():
    """Next-choice re-routing: the torch forward over the computing experts
    equals the C oracle's, gradcheck holds, and an expert that computes no
    slot gets no gradient while the router still does through the gates."""
    L = random_layer(11, T=12, d=6, h=5, E=5, k=2, act=SWIGLU, bias=True)
    L.b_gate = np.asarray([1.5, 1.0, 0, 0, 0], np.float32)
    idx, _, sc = oracle.route(L, want_scores=True)
    assign = oracle.capacity_reroute(L.cfg, idx, sc, 4)
    keep = oracle.capacity_keep(L.cfg, idx, 4)
    assert ((keep == 0) & (assign >= 0)).any()
    p = B.params(L)
    y, _, _, _ = B.forward(L, p, idx, assign=assign)
    yc, _, _ = oracle.forward_tokens(L, range(12), assign=assign)
    np.testing.assert_allclose(y.detach().numpy(), yc, rtol=1e-6, atol=1e-7 * np.abs(yc).max())
    dy = torch.from_numpy(np.random.default_rng(12).standard_normal((12, 6)))
    names = list(p)

    def f(*ts):
        return B.loss(L, dict(zip(names, ts)), idx, dy, None, 0.2, assign)

    assert torch.autograd.gradcheck(f, tuple(p[n] for n in names), eps=1e-6, atol=1e-6, rtol=1e-5)
    g = B.backward(L, dy.numpy(), importance_weight=0.2, idx=idx, assign=assign)
    for e in range(5):
        if not (assign == e).any():
            assert np.all(g["w_up"][e] == 0) and np.all(g["w_down"][e] == 0)
    assert np.abs(g["w_gate"]).max() > 0


def _noisy_layer(seed, T=9, d=6, h=5, E=5, k=2, S=0):
    L = random_layer(seed, T=T, d=d, h=h, E=E, k=k, act=SWIGLU, bias=True, S=S)
    rng = np.random.default_rng(seed + 100)
    L.w_noise = (rng.standard_normal((E, d)) * 0.4).astype(np.float32)
    noise = rng.standard_normal((T, E)).astype(np.float32)
    return L, noise


def test_noisy_forward_matches_the_c_oracle():
    """The torch noisy forward: gate values, and the smooth Load equal to
    the sum over tokens of the C oracle's P(x, i)."""
    L, noise = _noisy_layer(40, T=30, E=6, k=2)
    idx, kth = B.noisy_selection(L, noise)
    r = oracle.route_noisy(L, noise)
    p = B.params(L)
    _, g, _, load = B.forward(L, p, idx, noisy=dict(noise=noise, kth=kth))
    np.testing.assert_allclose(g.detach().numpy(), r["w"], rtol=1e-6)
    np.testing.assert_allclose(load.detach().numpy(), r["p"].sum(0), rtol=1e-6)


@pytest.mark.parametrize("k,E,S,imp_w,load_w", [(2, 5, 0, 0.0, 0.6), (2, 5, 1, 0.3, 0.4),
                                                (1, 4, 0, 0.2, 1.0), (3, 3, 0, 0.0, 0.5)])
def test_noisy_gradients_match_finite_differences(k, E, S, imp_w, load_w):
    """gradcheck of <dy, y> + w_imp CV^2(Importance) + w_load CV^2(Load)
    for the noisy gate, every input including W_noise (k = E: the Load is
    constant)."""
    L, noise = _noisy_layer(41 + k + E, E=E, k=k, S=S)
    idx, kth = B.noisy_selection(L, noise)
    noisy = dict(noise=noise, kth=kth)
    dy = torch.from_numpy(np.random.default_rng(5).standard_normal((L.cfg.T, L.cfg.d)))
    p = B.params(L)
    names = list(p)

    def f(*ts):
        return B.loss(L, dict(zip(names, ts)), idx, dy, None, imp_w, None, noisy, load_w)

    assert torch.autograd.gradcheck(f, tuple(p[n] for n in names), eps=1e-6, atol=1e-6, rtol=1e-5)


def test_noise_free_noisy_gate_is_the_clean_gate():
    """Zero draws: H = s, so the selection, the output gradients and the
    router's are the clean gate's, and W_noise gets no gradient from y (only
    the Load term reaches it, through the Softplus scales)."""
    L, noise = _noisy_layer(45, T=12, E=5, k=2)
    zero = np.zeros_like(noise)
    dy = np.random.default_rng(6).standard_normal((12, 6))
    gn = B.backward(L, dy, importance_weight=0.3, noise=zero, load_weight=0.0)
    gc = B.backward(L, dy, importance_weight=0.3)
    for n in gc:
        if n != "w_noise":
            np.testing.assert_allclose(gn[n], gc[n], rtol=1e-12, atol=1e-14)
    assert np.all(gn["w_noise"] == 0) and np.all(gc["w_noise"] == 0)
    gl = B.backward(L, dy, importance_weight=0.3, noise=zero, load_weight=0.5)
    assert np.abs(gl["w_noise"]).max() > 0


@pytest.mark.parametrize("act,S,gate,imp_w", [(SWIGLU, 1, 0, 0.4), (GELU, 0, 0, 0.3),
                                              (SWIGLU, 0, 1, 0.2), (SWIGLU, 0, 2, 0.5)])
def test_gradient_slices_equal_the_whole_graph(act, S, gate, imp_w):
    """The slices used at sizes too large for the whole graph: dx rows of a
    token subset (Importance linearised at the whole batch) and the weight
    gradients of some hidden units of one expert equal the corresponding
    entries of backward()."""
    L = random_layer(50 + gate, T=40, d=8, h=12, E=5, k=2, act=act, S=S, bias=True,
                     expert_bias=(act == GELU), gate=gate)
    dy = np.random.default_rng(51).standard_normal((40, 8))
    full = B.backward(L, dy, importance_weight=imp_w)
    toks = [0, 7, 19, 39]
    np.testing.assert_allclose(B.dx_rows(L, dy, toks, imp_w), full["x"][toks],
                               rtol=1e-10, atol=1e-12)
    units = np.array([0, 5, 11])
    for e in list(range(5)) + ([5] if S else []):
        g = B.expert_unit_grads(L, dy, e, units)
        up = full["w_up_shared"][0] if e == 5 else full["w_up"][e]
        down = full["w_down_shared"][0] if e == 5 else full["w_down"][e]
        if act == SWIGLU:
            np.testing.assert_allclose(g["w_up"][0], up[units], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(g["w_up"][1], up[units + 12], rtol=1e-10, atol=1e-12)
        else:
            np.testing.assert_allclose(g["w_up"], up[units], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(g["b_up"], full["b_up"][e][units], rtol=1e-10,
                                       atol=1e-12)
        np.testing.assert_allclose(g["w_down"], down[:, units], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("k,E", [(2, 5), (3, 3)])
def test_noisy_slices_equal_the_whole_graph(k, E):
    """The slices with the noisy gate: Importance and the smooth Load
    linearised at the whole batch give the whole graph's dx rows; the
    hidden-unit slices its expert weight gradients."""
    L, noise = _noisy_layer(60 + E, T=30, E=E, k=k)
    dy = np.random.default_rng(61).standard_normal((30, 6))
    full = B.backward(L, dy, importance_weight=0.3, noise=noise, load_weight=0.7)
    toks = [0, 11, 29]
    got = B.dx_rows(L, dy, toks, 0.3, noise=noise, load_weight=0.7)
    np.testing.assert_allclose(got, full["x"][toks], rtol=1e-10, atol=1e-12)
    units = np.array([0, 4])
    for e in range(E):
        g = B.expert_unit_grads(L, dy, e, units, noise=noise)
        np.testing.assert_allclose(g["w_up"][0], full["w_up"][e][units], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["w_up"][1], full["w_up"][e][units + 5], rtol=1e-10,
                                   atol=1e-12)
        np.testing.assert_allclose(g["w_down"], full["w_down"][e][:, units], rtol=1e-10,
                                   atol=1e-12)


def test_slot_outputs_are_the_expert_ffns():
    """oracle.slot_outputs (C, float64) row by row against the torch float64
    expert FFNs (written separately in oracle/backward.py), and the gated
    sum of the slots against the C forward; a dropped slot (-1) is zero."""
    for act, S, eb in ((SWIGLU, 1, False), (GELU, 0, True)):
        L = _layer(70, act, S, expert_bias=eb, T=20, d=12, h=10, E=6, k=3)
        idx, w, _ = oracle.route(L)
        toks = [0, 5, 19]
        ys = oracle.slot_outputs(L, toks, idx)
        p = {n: t.detach() for n, t in B.params(L).items()}
        for r, t in enumerate(toks):
            for j in range(3):
                ref = B._ffn(L.cfg, p, int(idx[t, j]), p["x"][t:t + 1])[0].numpy()
                np.testing.assert_allclose(ys[r, j], ref, rtol=1e-12, atol=1e-14)
        yc, _, _ = oracle.forward_tokens(L, toks)
        comb = np.einsum("tj,tjd->td", w[toks], ys)
        if S:
            comb += np.stack([oracle.expert(L, 6, B._f64(L.x)[t].numpy()) for t in toks])
        np.testing.assert_allclose(comb, yc, rtol=1e-12, atol=1e-14)
        dropped = np.where(np.arange(20 * 3).reshape(20, 3) % 4 == 1, -1, idx)
        yd = oracle.slot_outputs(L, toks, dropped)
        for r, t in enumerate(toks):
            for j in range(3):
                if dropped[t, j] < 0:
                    assert np.all(yd[r, j] == 0)
                else:
                    assert np.array_equal(yd[r, j], ys[r, j])


@pytest.mark.parametrize("gate,imp_w,policy", [(0, 0.4, None), (1, 0.3, None), (2, 0.5, None),
                                               (0, 0.2, "drop"), (0, 0.3, "next-choice")])
def test_router_gradient_slice_equals_the_whole_graph(gate, imp_w, policy):
    """The router's weight gradients from the slots' expert outputs held
    fixed equal those of backward() (the whole graph, pinned by gradcheck),
    for every gate mode and under a capacity with either overflow policy."""
    L = random_layer(80 + gate, T=40, d=8, h=12, E=5, k=2, act=SWIGLU, S=1, bias=True,
                     gate=gate)
    dy = np.random.default_rng(81).standard_normal((40, 8))
    idx, _, sc = oracle.route(L, want_scores=True)
    keep = assign = None
    experts = idx
    if policy == "drop":
        keep = oracle.capacity_keep(L.cfg, idx, 12)
        assert 0 < keep.sum() < keep.size
        experts = np.where(keep.reshape(40, 2) != 0, idx, -1)
    elif policy == "next-choice":
        assign = oracle.capacity_reroute(L.cfg, idx, sc, 12)
        assert np.any(assign.reshape(40, 2) != idx)
        experts = assign
    full = B.backward(L, dy, keep, imp_w, idx=idx, assign=assign)
    got = B.router_grads(L, B.slot_dy_products(L, dy, experts, chunk=16), imp_w, idx=idx)
    assert set(got) == {"w_gate", "b_gate"}
    for n in got:
        np.testing.assert_allclose(got[n], full[n], rtol=1e-10, atol=1e-12)


def test_noisy_router_gradient_slice_equals_the_whole_graph():
    """The same with the noisy gate: W_noise, W_g and b_g through the kept
    softmax of H and the smooth Load."""
    L, noise = _noisy_layer(85, T=30, E=5, k=2, S=1)
    dy = np.random.default_rng(86).standard_normal((30, 6))
    full = B.backward(L, dy, importance_weight=0.3, noise=noise, load_weight=0.7)
    sel = B.noisy_selection(L, noise)
    got = B.router_grads(L, B.slot_dy_products(L, dy, sel[0]), 0.3, noise=noise,
                         load_weight=0.7, selection=sel)
    assert set(got) == {"w_gate", "b_gate", "w_noise"}
    for n in got:
        np.testing.assert_allclose(got[n], full[n], rtol=1e-10, atol=1e-12)
