"""Pins of the CPU oracle to facts other than its own code.

Each test names what fixes the expected value: a number printed on the
pages (tests/golden/pages_pins.json), a closed form, an invariant, a
special case that reduces to a library routine (numpy/scipy/torch), or
brute force on tiny inputs.  Page names are the titles of the source pages.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import synthetic
from helpers import BF16, F32, GELU, SWIGLU, layer, random_layer

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "pages_pins.json")))


def _identity_router(scores, k):
    """A layer whose router scores are exactly ``scores``: x = scores and
    W_g = I, so every product is exact and every added term is +-0."""
    s = np.asarray(scores, np.float32)
    T, E = s.shape
    return layer(T, E, 4, E, k, x=s, w_gate=np.eye(E, dtype=np.float32),
                 w_up=np.zeros((E, 4, E)), w_down=np.zeros((E, E, 4)))


# ---------------------------------------------------------------- routing --

def test_router_worked_example(oracle_lib):
    """The techfeed summary's router example: scores over 6 experts pick
    indices 4 and 2; the two kept weights are the closed-form 2-way
    softmax sigma(l4 - l2)."""
    g = GOLD["router_example"]
    L = _identity_router([g["scores"]], g["k"])
    idx, w, sc = oracle_lib.route(L, want_scores=True)
    assert sc[0].tolist() == np.float32(g["scores"]).tolist()
    assert idx[0].tolist() == g["expected_indices"]
    l4, l2 = float(np.float32(0.5106)), float(np.float32(0.4254))
    assert w[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(l2 - l4)), rel=1e-15)
    assert w[0, 1] == pytest.approx(1.0 / (1.0 + math.exp(l4 - l2)), rel=1e-15)
    assert w[0, 0] == pytest.approx(0.5212871, abs=5e-8)


@pytest.mark.parametrize("E,k", [(6, 2), (8, 1), (8, 8), (32, 4), (256, 8)])
def test_keep_topk_is_stable_descending_sort(oracle_lib, E, k):
    """KeepTopK = first k of a stable descending sort (lower index first on
    ties): compared with numpy's stable argsort; many forced ties."""
    rng = np.random.default_rng(E * 31 + k)
    s = (np.round(rng.standard_normal((200, E)) * 2) / 2).astype(np.float32)
    s[0] = 0.0
    s[1, :] = -0.0
    s[1, ::3] = 0.0          # +0 and -0 compare equal
    L = _identity_router(s, k)
    idx, w, _ = oracle_lib.route(L)
    ref = np.argsort(-s.astype(np.float64), axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, ref)
    assert idx[0].tolist() == list(range(k))
    assert idx[1].tolist() == list(range(k))


def test_ties_zero_input_and_duplicate_rows(oracle_lib):
    """x = 0 gives equal scores: indices 0..k-1 and weights 1/k.  Two equal
    router rows (experts 3 and 5) that beat the rest keep the order 3, 5."""
    E, d, k = 8, 16, 3
    rng = np.random.default_rng(1)
    wg = rng.standard_normal((E, d)).astype(np.float32) * 0.1
    wg[5] = wg[3]
    x = np.zeros((2, d), np.float32)
    x[1] = wg[3] * 50
    L = layer(2, d, 4, E, k, x=x, w_gate=wg, w_up=np.zeros((E, 4, d)),
              w_down=np.zeros((E, d, 4)))
    idx, w, sc = oracle_lib.route(L, want_scores=True)
    assert idx[0].tolist() == [0, 1, 2]
    assert np.all(w[0] == 1.0 / 3.0)
    assert sc[1, 3] == sc[1, 5]
    assert idx[1, :2].tolist() == [3, 5]


def test_softmax_closed_forms(oracle_lib):
    """k = 1 gives weight exactly 1; k = 2 is sigma(l0 - l1); k = E is the
    dense softmax gate softmax(x W_g) of the Qiita summary (scipy)."""
    rng = np.random.default_rng(2)
    s = rng.standard_normal((50, 6)).astype(np.float32) * 3
    idx1, w1, _ = oracle_lib.route(_identity_router(s, 1))
    assert np.all(w1 == 1.0)
    idx2, w2, _ = oracle_lib.route(_identity_router(s, 2))
    l0 = np.take_along_axis(s, idx2[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(s, idx2[:, 1:], 1)[:, 0].astype(np.float64)
    np.testing.assert_allclose(w2[:, 0], 1 / (1 + np.exp(l1 - l0)), rtol=1e-14)
    idx6, w6, _ = oracle_lib.route(_identity_router(s, 6))
    dense = scipy.special.softmax(s.astype(np.float64), axis=1)
    np.testing.assert_allclose(w6, np.take_along_axis(dense, idx6, 1), rtol=1e-13)


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_kept_weights_sum_to_one_and_descend(oracle_lib, k):
    L = random_layer(3, T=300, d=40, h=8, E=16, k=k, bias=True)
    idx, w, _ = oracle_lib.route(L)
    assert np.all(np.abs(w.sum(1) - 1.0) <= k * 2.0 ** -52 * 4)
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == k for r in idx.tolist())


def test_router_scores_exact_integer_products(oracle_lib):
    """Small integers: every partial sum is exact in float32, so the scores
    equal the integer matrix product (numpy int64) plus the bias."""
    rng = np.random.default_rng(4)
    T, d, E = 20, 24, 7
    x = rng.integers(-8, 9, (T, d))
    wg = rng.integers(-8, 9, (E, d))
    b = rng.integers(-50, 50, E)
    L = layer(T, d, 4, E, 2, x=x, w_gate=wg, b_gate=b,
              w_up=np.zeros((E, 4, d)), w_down=np.zeros((E, d, 4)))
    _, _, sc = oracle_lib.route(L, want_scores=True)
    assert np.array_equal(sc, (x @ wg.T + b).astype(np.float32))


def test_router_scores_fused_multiply_add_per_term(oracle_lib):
    """Reading of the Go Route loop: one fused multiply-add per term.  With
    s = -1 after term 0, term 1 adds (1 + 2^-12)^2 = 1 + 2^-11 + 2^-24
    without rounding the product first: the score is 2^-11 + 2^-24 (an
    unfused multiply-add would give 2^-11)."""
    a = 1.0 + 2.0 ** -12
    L = layer(1, 2, 4, 2, 1, x=[[1.0, a]], w_gate=[[-1.0, a], [0.0, 0.0]],
              w_up=np.zeros((2, 4, 2)), w_down=np.zeros((2, 2, 4)))
    _, _, sc = oracle_lib.route(L, want_scores=True)
    assert float(sc[0, 0]) == 2.0 ** -11 + 2.0 ** -24


def test_router_scores_ascending_order(oracle_lib):
    """Terms are added in ascending i: 2^24 + 1 rounds back to 2^24 and the
    last term cancels it, so the score is 0 (descending order would give 1)."""
    L = layer(1, 3, 4, 2, 1, x=[[2.0 ** 24, 1.0, -(2.0 ** 24)]],
              w_gate=[[1.0, 1.0, 1.0], [0.0, 0.0, 0.0]],
              w_up=np.zeros((2, 4, 3)), w_down=np.zeros((2, 3, 4)))
    _, _, sc = oracle_lib.route(L, want_scores=True)
    assert float(sc[0, 0]) == 0.0


def test_router_scores_within_float32_error_bound(oracle_lib):
    """|score - exact dot| <= gamma_d * sum|x_i w_i| + |bias| u (standard
    error bound of a length-d float32 recursive sum)."""
    L = random_layer(5, T=64, d=512, h=8, E=12, k=2, dtype=BF16, bias=True)
    _, _, sc = oracle_lib.route(L, want_scores=True)
    xf = (L.x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wg = L.w_gate.astype(np.float64)
    exact = xf @ wg.T + L.b_gate.astype(np.float64)
    u = 2.0 ** -24
    gam = (513 * u) / (1 - 513 * u)
    bound = gam * (np.abs(xf) @ np.abs(wg).T + np.abs(L.b_gate))
    assert np.all(np.abs(sc - exact) <= bound)


def test_non_finite_input_rejected(oracle_lib):
    L = random_layer(6, T=4, d=8, h=8, E=4, k=2)
    L.x[2, 3] = np.nan
    with pytest.raises(FloatingPointError):
        oracle_lib.route(L)


# -------------------------------------------------- counts / permutation --

def test_counts_importance_and_permutation(oracle_lib):
    """Counts = histogram of the kept indices (np.bincount), summing to T*k;
    Importance = per-expert sum of the kept weights (sums to T); the
    grouping is numpy's stable argsort of the flat index array."""
    L = random_layer(7, T=333, d=32, h=8, E=12, k=3, bias=True)
    c = L.cfg
    idx, w, _ = oracle_lib.route(L)
    cnt, imp = oracle_lib.counts(c, idx, w)
    assert np.array_equal(cnt, np.bincount(idx.ravel(), minlength=c.E))
    assert cnt.sum() == c.T * c.k
    np.testing.assert_allclose(
        imp, np.bincount(idx.ravel(), weights=w.ravel(), minlength=c.E), rtol=1e-13)
    assert imp.sum() == pytest.approx(c.T, rel=1e-13)
    off, src, pos = oracle_lib.permute(c, idx)
    order = np.argsort(idx.ravel(), kind="stable")
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]))
    assert np.array_equal(src, order // c.k)
    assert np.array_equal(pos[order], np.arange(c.T * c.k))


def test_permutation_with_empty_experts(oracle_lib):
    L = _identity_router(np.tile(np.float32([5, 4, 0, 0, 3, 0]), (9, 1)), 2)
    idx, w, _ = oracle_lib.route(L)
    off, src, pos = oracle_lib.permute(L.cfg, idx)
    assert off.tolist() == [0, 9, 18, 18, 18, 18, 18]
    assert src.tolist() == list(range(9)) * 2


# ----------------------------------------------------------- expert FFNs --

def _int_gelu_layer(dtype, seed):
    """GELU experts whose pre-activations are all multiples of 64: in double,
    erf(+-45.25) is exactly +-1, so GELU(a) = max(a, 0) exactly and the FFN
    reduces to integer matrix products (numpy int64)."""
    rng = np.random.default_rng(seed)
    E, d, h, T = 3, 6, 10, 5
    x = rng.integers(-1, 2, (T, d))
    w1 = rng.integers(-2, 3, (E, h, d)) * 64
    b1 = rng.integers(-2, 3, (E, h)) * 64
    w2 = rng.integers(-3, 4, (E, d, h))
    b2 = rng.integers(-9, 10, (E, d))
    L = layer(T, d, h, E, 2, GELU, dtype, x=x, w_gate=np.ones((E, d)),
              w_up=w1, w_down=w2, b_up=b1, b_down=b2)
    return L, x, w1, b1, w2, b2


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_gelu_expert_reduces_to_integer_matmul(oracle_lib, dtype):
    L, x, w1, b1, w2, b2 = _int_gelu_layer(dtype, 8)
    for e in range(3):
        for t in range(5):
            ref = w2[e] @ np.maximum(w1[e] @ x[t] + b1[e], 0) + b2[e]
            got = oracle_lib.expert(L, e, x[t].astype(np.float64))
            assert np.array_equal(got, ref.astype(np.float64)), (e, t)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_swiglu_expert_reduces_to_integer_matmul(oracle_lib, dtype):
    """SwiGLU with packed [2h, d] gate/up rows.  x in {0, 1}, gate weights in
    {0, 64, -2048} with d = 6: every gate pre-activation is 0, >= 64 or
    <= -1728, where silu(g) is exactly g, g, or -0 in double, so
    H = max(gate, 0) * up and y = W2 H are integer matrix products."""
    rng = np.random.default_rng(9)
    E, d, h, T = 2, 6, 5, 7
    x = rng.integers(0, 2, (T, d))
    gate = rng.choice([0, 64, -2048], size=(E, h, d), p=[0.4, 0.45, 0.15])
    up = rng.integers(-3, 4, (E, h, d))
    w2 = rng.integers(-3, 4, (E, d, h))
    L = layer(T, d, h, E, 1, SWIGLU, dtype, x=x, w_gate=np.ones((E, d)),
              w_up=np.concatenate([gate, up], axis=1), w_down=w2)
    for e in range(E):
        for t in range(T):
            hid = np.maximum(gate[e] @ x[t], 0) * (up[e] @ x[t])
            got = oracle_lib.expert(L, e, x[t].astype(np.float64))
            assert np.array_equal(got, (w2[e] @ hid).astype(np.float64)), (e, t)


def test_activation_values(oracle_lib):
    """GELU(1) = Phi(1); SwiGLU(1) = sigmoid(1); SwiGLU(ln 3) = (3/4) (ln 3)^2,
    all through 1x1 experts."""
    Lg = layer(1, 1, 1, 1, 1, GELU, x=[[1.0]], w_gate=[[1.0]],
               w_up=[[[1.0]]], w_down=[[[1.0]]])
    phi1 = 0.5 * (1 + math.erf(1 / math.sqrt(2)))
    assert oracle_lib.expert(Lg, 0, np.array([1.0]))[0] == pytest.approx(phi1, rel=1e-15)
    assert phi1 == pytest.approx(0.8413447460685429, rel=1e-15)
    Ls = layer(1, 1, 1, 1, 1, SWIGLU, x=[[1.0]], w_gate=[[1.0]],
               w_up=[[[1.0]], [[1.0]]], w_down=[[[1.0]]])
    ln3 = math.log(3.0)
    assert oracle_lib.expert(Ls, 0, np.array([1.0]))[0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)
    assert oracle_lib.expert(Ls, 0, np.array([ln3]))[0] == pytest.approx(0.75 * ln3 * ln3, rel=1e-14)


@pytest.mark.parametrize("act", [GELU, SWIGLU])
def test_single_expert_top1_is_plain_ffn(oracle_lib, act):
    """The Go chapter's boundary check: 1 expert, top-1 equals a plain FFN.
    The plain FFN here is torch's Linear/GELU/SiLU in float64."""
    g = GOLD["single_expert_is_ffn"]
    L = random_layer(10, T=9, d=12, h=20, E=g["E"], k=g["k"], act=act,
                     expert_bias=(act == GELU))
    y, idx, w = oracle_lib.forward_tokens(L, range(9))
    assert np.all(idx == 0) and np.all(w == 1.0)
    X = torch.tensor(L.x, dtype=torch.float64)
    W1 = torch.tensor(L.w_up[0], dtype=torch.float64)
    W2 = torch.tensor(L.w_down[0], dtype=torch.float64)
    if act == GELU:
        hid = torch.nn.functional.gelu(
            torch.nn.functional.linear(X, W1, torch.tensor(L.b_up[0], dtype=torch.float64)))
        ref = torch.nn.functional.linear(hid, W2, torch.tensor(L.b_down[0], dtype=torch.float64))
    else:
        hdim = L.cfg.h
        hid = torch.nn.functional.silu(X @ W1[:hdim].T) * (X @ W1[hdim:].T)
        ref = hid @ W2.T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("act,S", [(GELU, 0), (SWIGLU, 0), (SWIGLU, 1)])
def test_sparse_forward_equals_dense_gated_sum(oracle_lib, act, S):
    """y = sum over ALL experts of G_i * E_i(x), with G = softmax(KeepTopK)
    built densely (-inf outside the top k, scipy softmax): the sparse token
    loop that skips zero gates gives the same result (Qiita summary,
    'Sparsely-Gated MoE layer formula')."""
    L = random_layer(11, T=6, d=10, h=14, E=5, k=2, act=act, S=S, bias=True)
    c = L.cfg
    y, idx, w = oracle_lib.forward_tokens(L, range(c.T))
    _, _, sc = oracle_lib.route(L, want_scores=True)
    for t in range(c.T):
        keep = np.full(c.E, -np.inf)
        top = np.argsort(-sc[t].astype(np.float64), kind="stable")[:c.k]
        keep[top] = sc[t, top]
        G = scipy.special.softmax(keep)
        xr = L.x[t].astype(np.float64)
        dense = sum(G[i] * oracle_lib.expert(L, i, xr) for i in range(c.E))
        if S:
            dense = dense + oracle_lib.expert(L, c.E, xr)
        np.testing.assert_allclose(y[t], dense, rtol=1e-12, atol=1e-14)
        assert np.count_nonzero(G) == c.k


def test_output_scales_exactly_with_down_projection(oracle_lib):
    L = random_layer(12, T=7, d=16, h=24, E=4, k=2, act=SWIGLU)
    y1, _, _ = oracle_lib.forward_tokens(L, range(7))
    L.w_down = np.ascontiguousarray(L.w_down * np.float32(8.0))
    y8, _, _ = oracle_lib.forward_tokens(L, range(7))
    assert np.array_equal(y8, 8.0 * y1)


def test_zero_down_projection_gives_bias(oracle_lib):
    """W2 = 0: every expert outputs b2, and the kept weights sum to 1."""
    L = random_layer(13, T=5, d=8, h=16, E=4, k=2, expert_bias=True)
    L.w_down = np.zeros_like(L.w_down)
    L.b_down = np.ascontiguousarray(np.tile(np.float32([1, 2, 3, 4, 5, 6, 7, 8]), (4, 1)))
    y, _, _ = oracle_lib.forward_tokens(L, range(5))
    np.testing.assert_allclose(y, np.tile(np.arange(1, 9.0), (5, 1)), rtol=1e-15)


# ------------------------------------------------------------ statistics --

def test_load_balance_loss_ends_and_cv(oracle_lib):
    """Go chapter: loss 1 when uniform, N when concentrated, 0 when empty.
    With population variance, loss = 1 + CV^2(Load) for any counts."""
    g = GOLD["load_balance_ends"]
    for N in (2, 6, 8, 256):
        assert oracle_lib.load_stats(np.full(N, 5))[2] == g["uniform"]
        one = np.zeros(N, np.int32)
        one[N // 3] = 17
        assert oracle_lib.load_stats(one)[2] == pytest.approx(N, rel=1e-15)
        assert oracle_lib.load_stats(np.zeros(N, np.int32))[2] == 0.0
    rng = np.random.default_rng(14)
    for _ in range(20):
        cnt = rng.integers(0, 100, 16)
        cv_imp, cv_load, lb = oracle_lib.load_stats(cnt, cnt * 0.5)
        assert lb == pytest.approx(1.0 + cv_load, rel=1e-13)
        m = cnt.mean()
        assert cv_load == pytest.approx(cnt.var() / m / m, rel=1e-12)
        assert cv_imp == pytest.approx(cv_load, rel=1e-12)
    assert oracle_lib.load_stats(np.int32([1, 0, 0, 0]))[1] == pytest.approx(3.0)


def test_parameter_accounting(oracle_lib):
    """Go chapter, 'Parameter accounting': at 8 experts / top-2 the experts'
    total is 4x the active count; Total = d*E + E*P_e, Active = d*E + k*P_e."""
    from synthetic import MIXTRAL, TINY
    g = GOLD["expert_total_over_active"]
    for cfg in (TINY, MIXTRAL):
        assert (cfg.E, cfg.k) == (g["E"], g["k"])
        tot, act = oracle_lib.param_counts(cfg)
        router = cfg.d * cfg.E
        assert (tot - router) == g["ratio"] * (act - router)
    tot, act = oracle_lib.param_counts(TINY)
    assert (tot - 512, act - 512) == (262144, 65536)
    tot, act = oracle_lib.param_counts(MIXTRAL)
    assert (tot - 4096 * 8, act - 4096 * 8) == (1409286144, 352321536)


def test_invalid_configs_rejected(oracle_lib):
    L = random_layer(15, T=4, d=8, h=8, E=4, k=2)
    L.cfg = L.cfg.with_(k=5)
    with pytest.raises(ValueError):
        oracle_lib.route(L)
    L.cfg = L.cfg.with_(k=0)
    with pytest.raises(ValueError):
        oracle_lib.route(L)


# ---- expert capacity (Go chapter, "What was simplified": an expert accepts
# at most C tokens, the overflow is dropped) ----

def _routing(seed, T, E, k):
    rng = np.random.default_rng(seed)
    # k distinct experts per token, skewed towards low indices
    p = np.exp(-0.3 * np.arange(E))
    p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("C", [1, 3, 7, 40])
def test_capacity_keeps_first_C_assignments_in_flat_order(oracle_lib, C):
    """keep = the first C flat indices t*k+j of each expert (numpy nonzero
    order), and an expert keeps min(n_e, C) assignments."""
    T, E, k = 60, 6, 2
    idx = _routing(C, T, E, k)
    c = synthetic.TINY.with_(T=T, E=E, k=k)
    keep = oracle_lib.capacity_keep(c, idx, C)
    ref = np.zeros(T * k, np.uint8)
    flat = idx.ravel()
    for e in range(E):
        ref[np.flatnonzero(flat == e)[:C]] = 1
    np.testing.assert_array_equal(keep, ref)
    n = np.bincount(flat, minlength=E)
    kept = np.bincount(flat[keep == 1], minlength=E)
    np.testing.assert_array_equal(kept, np.minimum(n, C))


def test_capacity_zero_or_large_keeps_everything(oracle_lib):
    L = random_layer(3, T=9, d=8, h=12, E=4, k=2, act=SWIGLU, S=1, bias=True)
    c = L.cfg
    idx, _, _ = oracle_lib.route(L)
    for C in (0, c.T * c.k):
        assert oracle_lib.capacity_keep(c, idx, C).all()
    y0, _, _ = oracle_lib.forward_tokens(L, range(c.T))
    y1, _, _ = oracle_lib.forward_tokens(L, range(c.T), keep=np.ones(c.T * c.k, np.uint8))
    np.testing.assert_array_equal(y0, y1)


def test_capacity_grouping_of_kept_rows(oracle_lib):
    """Kept rows grouped by expert in flat order (numpy lexsort), offsets =
    exclusive scan of min(n_e, C), pos = -1 exactly for dropped slots."""
    T, E, k, C = 50, 5, 3, 9
    idx = _routing(7, T, E, k)
    c = synthetic.TINY.with_(T=T, E=E, k=k)
    keep = oracle_lib.capacity_keep(c, idx, C)
    off, src, pos = oracle_lib.permute_keep(c, idx, keep)
    flat = idx.ravel()
    n = np.minimum(np.bincount(flat, minlength=E), C)
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(n)]))
    kept_f = np.flatnonzero(keep)
    order = kept_f[np.lexsort((kept_f, flat[kept_f]))]
    np.testing.assert_array_equal(src, order // k)
    ref_pos = np.full(T * k, -1, np.int32)
    ref_pos[order] = np.arange(order.size)
    np.testing.assert_array_equal(pos, ref_pos)


@pytest.mark.parametrize("S", [0, 1])
def test_dropped_slots_are_zeroed_gates_without_renormalisation(oracle_lib, S):
    """With a capacity the layer equals the dense gated sum in which the
    dropped experts' gates are set to 0 and the others keep their softmax
    values (scipy softmax over the kept k)."""
    L = random_layer(12, T=24, d=10, h=14, E=5, k=2, act=SWIGLU, S=S, bias=True)
    c = L.cfg
    idx, _, sc = oracle_lib.route(L, want_scores=True)
    keep = oracle_lib.capacity_keep(c, idx, 4)
    assert 0 < keep.sum() < c.T * c.k
    y, _, _ = oracle_lib.forward_tokens(L, range(c.T), keep=keep)
    for t in range(c.T):
        g = np.full(c.E, -np.inf)
        top = np.argsort(-sc[t].astype(np.float64), kind="stable")[:c.k]
        g[top] = sc[t, top]
        G = scipy.special.softmax(g)
        for j in range(c.k):
            if not keep[t * c.k + j]:
                G[top[j]] = 0.0
        xr = L.x[t].astype(np.float64)
        dense = sum(G[i] * oracle_lib.expert(L, i, xr) for i in range(c.E))
        if S:
            dense = dense + oracle_lib.expert(L, c.E, xr)
        np.testing.assert_allclose(y[t], dense, rtol=1e-12, atol=1e-14)


def test_token_with_every_slot_dropped(oracle_lib):
    """A token whose experts are all full adds no routed term: y = 0 without
    a shared expert (exactly), y = the shared expert with one."""
    for S in (0, 1):
        L = random_layer(5, T=6, d=8, h=8, E=2, k=2, act=SWIGLU, S=S)
        c = L.cfg
        idx, _, _ = oracle_lib.route(L)
        keep = oracle_lib.capacity_keep(c, idx, 1)   # E = k = 2: token 0 fills both
        assert keep[:2].all() and not keep[2:].any()
        y, _, _ = oracle_lib.forward_tokens(L, [4], keep=keep)
        if S:
            ref = oracle_lib.expert(L, c.E, L.x[4].astype(np.float64))
            np.testing.assert_array_equal(y[0], ref)
        else:
            np.testing.assert_array_equal(y[0], np.zeros(c.d))


# ---- next-choice re-routing of the overflow (Go chapter, "Design
# viewpoints", capacity factor: an overflowing token is dropped or handed to
# its next candidate).  Reading: one hop; the o-th overflowing slot of a token
# is offered to its o-th best expert outside its top k; experts take offers
# in flat order into the room the first round left ----

def _reroute(oracle_lib, scores, idx, C):
    s = np.asarray(scores, np.float32)
    idx = np.asarray(idx, np.int32).reshape(s.shape[0], -1)
    c = synthetic.TINY.with_(T=s.shape[0], E=s.shape[1], k=idx.shape[1])
    return oracle_lib.capacity_reroute(c, idx, s, C).tolist()


def test_reroute_worked_examples(oracle_lib):
    # every token prefers expert 0 (C = 1): token 1 moves to its second
    # choice 2, token 2 to its second choice 1
    assert _reroute(oracle_lib, [[3, 2, 1], [3, 1, 2], [3, 2, 1]], [0, 0, 0], 1) == [0, 2, 1]
    # two offers to the same expert: the earlier token takes the one place
    assert _reroute(oracle_lib, [[3, 2, 1]] * 3, [0, 0, 0], 1) == [0, 1, -1]
    # a token with both slots overflowing: slot 0 gets its best expert
    # outside the top 2 (expert 3, score 2), slot 1 the next one (expert 2)
    assert _reroute(oracle_lib, [[4, 3, 2, 1], [4, 3, 1, 2]], [[0, 1], [0, 1]], 1) == [0, 1, 3, 2]
    # equal candidate scores: the lower index first
    assert _reroute(oracle_lib, [[5, 1, 1, 1]] * 2, [0, 0], 1) == [0, 1]
    # the first round fills every expert before any offer: token 2's own
    # choice of expert 1 outranks token 1's offer to it, and the offer is
    # dropped (one hop: no third try)
    assert _reroute(oracle_lib, [[3, 1, 2], [3, 2, 1], [1, 3, 2]], [0, 0, 1], 1) == [0, -1, 1]


def _ranked_outside(scores_t, top):
    rest = [e for e in range(len(scores_t)) if e not in set(top)]
    return sorted(rest, key=lambda e: (-float(scores_t[e]), e))


@pytest.mark.parametrize("C", [12, 17, 25])
def test_reroute_against_brute_force(oracle_lib, C):
    """Re-implementation by rounds over Python lists of the reading, on
    skewed routings: kept slots unchanged, offers by ordinal, room left."""
    T, E, k = 40, 7, 3
    L = random_layer(20 + C, T=T, d=8, h=8, E=E, k=k, bias=True)
    L.b_gate = np.asarray([2.0, 1.5, 1.0, 0, 0, 0, 0], np.float32)   # skew to low experts
    c = L.cfg
    idx, _, sc = oracle_lib.route(L, want_scores=True)
    assign = oracle_lib.capacity_reroute(c, idx, sc, C)
    keep = oracle_lib.capacity_keep(c, idx, C)
    flat = idx.ravel()
    taken = np.minimum(np.bincount(flat, minlength=E), C)
    ref = np.where(keep == 1, flat, -1)
    offers = {}
    for t in range(T):
        cand = _ranked_outside(sc[t], idx[t])
        o = 0
        for j in range(k):
            f = t * k + j
            if keep[f]:
                continue
            offers[f] = cand[o] if o < len(cand) else -1
            o += 1
    for f in sorted(offers):
        e = offers[f]
        if e >= 0 and taken[e] < C:
            ref[f] = e
            taken[e] += 1
    np.testing.assert_array_equal(assign, ref)
    assert (keep == 0).any() and (assign[keep == 0] >= 0).any()
    # invariants: capacity honoured, re-routed experts outside the top k
    assert (np.bincount(assign[assign >= 0], minlength=E) <= C).all()
    for f in np.flatnonzero((keep == 0) & (assign >= 0)):
        assert assign[f] not in idx[f // k]


def test_reroute_degenerate_cases(oracle_lib):
    L = random_layer(21, T=30, d=8, h=8, E=4, k=2)
    c = L.cfg
    idx, _, sc = oracle_lib.route(L, want_scores=True)
    # no limit, or room for everything: every slot computed where it was routed
    for C in (0, c.T * c.k):
        np.testing.assert_array_equal(oracle_lib.capacity_reroute(c, idx, sc, C), idx.ravel())
    # E = k: no expert outside the top k, so re-routing is the drop rule
    L2 = random_layer(22, T=30, d=8, h=8, E=2, k=2)
    idx2, _, sc2 = oracle_lib.route(L2, want_scores=True)
    keep = oracle_lib.capacity_keep(L2.cfg, idx2, 7)
    np.testing.assert_array_equal(oracle_lib.capacity_reroute(L2.cfg, idx2, sc2, 7),
                                  np.where(keep == 1, idx2.ravel(), -1))


def test_assign_grouping(oracle_lib):
    """Rows grouped by computing expert in flat order (numpy lexsort); with
    the drop rule's assignment it is the kept grouping."""
    T, E, k, C = 50, 5, 3, 9
    idx = _routing(7, T, E, k)
    c = synthetic.TINY.with_(T=T, E=E, k=k)
    keep = oracle_lib.capacity_keep(c, idx, C)
    drop_assign = np.where(keep == 1, idx.ravel(), -1).astype(np.int32)
    for a, b in zip(oracle_lib.permute_assign(c, drop_assign),
                    oracle_lib.permute_keep(c, idx, keep)):
        np.testing.assert_array_equal(a, b)
    rng = np.random.default_rng(3)
    assign = rng.integers(-1, E, size=T * k).astype(np.int32)
    off, src, pos = oracle_lib.permute_assign(c, assign)
    live = np.flatnonzero(assign >= 0)
    order = live[np.lexsort((live, assign[live]))]
    np.testing.assert_array_equal(off, np.concatenate(
        [[0], np.cumsum(np.bincount(assign[live], minlength=E))]))
    np.testing.assert_array_equal(src, order // k)
    ref_pos = np.full(T * k, -1, np.int32)
    ref_pos[order] = np.arange(order.size)
    np.testing.assert_array_equal(pos, ref_pos)


@pytest.mark.parametrize("S", [0, 1])
def test_rerouted_forward_is_gated_sum_over_computing_experts(oracle_lib, S):
    """y_t = sum_j G_j E_{a_j}(x_t) (+ shared): the kept-k softmax values
    (scipy) applied to the expert that computes each slot."""
    L = random_layer(23, T=24, d=10, h=14, E=5, k=2, act=SWIGLU, S=S, bias=True)
    L.b_gate = np.asarray([1.5, 1.0, 0, 0, 0], np.float32)
    c = L.cfg
    idx, _, sc = oracle_lib.route(L, want_scores=True)
    assign = oracle_lib.capacity_reroute(c, idx, sc, 6)
    keep = oracle_lib.capacity_keep(c, idx, 6)
    assert ((keep == 0) & (assign >= 0)).any() and (assign < 0).any()
    y, _, _ = oracle_lib.forward_tokens(L, range(c.T), assign=assign)
    for t in range(c.T):
        top = np.argsort(-sc[t].astype(np.float64), kind="stable")[:c.k]
        G = scipy.special.softmax(sc[t, top].astype(np.float64))
        xr = L.x[t].astype(np.float64)
        ref = np.zeros(c.d)
        for j in range(c.k):
            e = assign[t * c.k + j]
            if e >= 0:
                ref = ref + G[j] * oracle_lib.expert(L, int(e), xr)
        if S:
            ref = ref + oracle_lib.expert(L, c.E, xr)
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-14)


# ---- gate modes.  bias-selects: the bias steers the selection only (Go
# chapter, section 3 and "Pros, cons and real examples": DeepSeek-V3 balances
# load through a bias instead of a loss); softmax-all: the softmax over all E
# scores weights the chosen experts as it is (techfeed summary, "The hardest
# part: making the router trainable"; k = 1 is the Switch Transformer gate) ----

def _with_gate(L, gate, b_gate="keep"):
    L.cfg = L.cfg.with_(gate=gate)
    if not isinstance(b_gate, str):
        L.b_gate = None if b_gate is None else np.asarray(b_gate, np.float32)
    return L


def test_bias_selects_worked_example(oracle_lib):
    """The techfeed scores with a bias lifting experts 0 (+2) and 1 (+1):
    both modes select [0, 1]; the default weights are sigma of the biased
    gap, bias-selects weights sigma of the unbiased gap."""
    g = GOLD["router_example"]
    s = np.float32(g["scores"])
    b = np.float32([2, 1, 0, 0, 0, 0])
    l0, l1 = float(s[0]), float(s[1])
    for gate, gap in ((synthetic.GATE_TOPK_SOFTMAX, float(np.float32(l0 + 2)) - float(np.float32(l1 + 1))),
                      (synthetic.GATE_BIAS_SELECTS, l0 - l1)):
        L = _with_gate(_identity_router([s], 2), gate, b)
        idx, w, sc = oracle_lib.route(L, want_scores=True)
        assert idx[0].tolist() == [0, 1]
        assert sc[0].tolist() == (s + b).tolist()
        assert w[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-gap)), rel=1e-15)
        assert w[0, 1] == pytest.approx(1.0 / (1.0 + math.exp(gap)), rel=1e-15)


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_bias_selects_weights_are_unbiased_softmax(oracle_lib, k):
    """Same selection as the default mode; weights = scipy softmax of the
    scores the same router gives without its bias, at the kept experts.
    Without a bias the two modes agree exactly."""
    L = random_layer(21, T=40, d=24, h=8, E=8, k=k, act=SWIGLU, bias=True)
    idx0, _, sc = oracle_lib.route(L, want_scores=True)
    b = L.b_gate
    _with_gate(L, synthetic.GATE_BIAS_SELECTS)
    idx1, w1, sc1 = oracle_lib.route(L, want_scores=True)
    np.testing.assert_array_equal(idx1, idx0)
    np.testing.assert_array_equal(sc1, sc)
    _with_gate(L, synthetic.GATE_TOPK_SOFTMAX, None)
    _, _, raw = oracle_lib.route(L, want_scores=True)
    assert not np.array_equal(raw, sc)
    ref = scipy.special.softmax(np.take_along_axis(raw, idx1, 1).astype(np.float64), axis=1)
    np.testing.assert_allclose(w1, ref, rtol=1e-13, atol=0)
    # no bias: the modes coincide
    idx_a, w_a, _ = oracle_lib.route(L)
    _with_gate(L, synthetic.GATE_BIAS_SELECTS, None)
    idx_b, w_b, _ = oracle_lib.route(L)
    np.testing.assert_array_equal(idx_a, idx_b)
    np.testing.assert_array_equal(w_a, w_b)
    del b


def test_softmax_all_closed_forms(oracle_lib):
    """Techfeed scores: k = 1 gives p_max = 1 / sum_e exp(s_e - s_max) (the
    Switch gate), k = 2 gives p_4 and p_2 from the full softmax (their sum
    below 1), k = E gives the whole softmax in descending order (sum 1)."""
    s = np.float64(np.float32(GOLD["router_example"]["scores"]))
    z = sum(math.exp(v - s.max()) for v in s)
    for k in (1, 2, 6):
        L = _with_gate(_identity_router([np.float32(s)], k), synthetic.GATE_SOFTMAX_ALL)
        idx, w, _ = oracle_lib.route(L)
        assert idx[0, :2].tolist() == [4, 2][:k]
        for j in range(k):
            assert w[0, j] == pytest.approx(math.exp(s[idx[0, j]] - s.max()) / z, rel=1e-15)
        if k == 6:
            assert w[0].sum() == pytest.approx(1.0, rel=1e-15)
        else:
            assert w[0].sum() < 1.0


@pytest.mark.parametrize("k", [1, 3, 8])
def test_softmax_all_against_scipy_and_kept_ratios(oracle_lib, k):
    """Weights = scipy softmax over all E (biased) scores read at the kept
    experts; their ratios equal those of the default (renormalised) mode."""
    L = random_layer(22, T=50, d=16, h=8, E=8, k=k, act=GELU, bias=True)
    idx0, w0, sc = oracle_lib.route(L, want_scores=True)
    _with_gate(L, synthetic.GATE_SOFTMAX_ALL)
    idx2, w2, _ = oracle_lib.route(L)
    np.testing.assert_array_equal(idx2, idx0)
    p = scipy.special.softmax(sc.astype(np.float64), axis=1)
    np.testing.assert_allclose(w2, np.take_along_axis(p, idx2, 1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(w2 / w2.sum(1, keepdims=True), w0, rtol=1e-13, atol=0)


@pytest.mark.parametrize("S", [0, 1])
def test_softmax_all_with_every_expert_is_dense_softmax_gate(oracle_lib, S):
    """k = E: the layer is the dense softmax-gated mixture sum_e softmax(s)_e
    E_e(x) (Qiita summary, "Sparsely-Gated MoE layer formula" with the
    plain softmax gate); k < E: the same sum over the kept experts only."""
    for k in (5, 2):
        L = random_layer(23, T=5, d=10, h=12, E=5, k=k, act=SWIGLU, S=S, bias=True,
                         gate=synthetic.GATE_SOFTMAX_ALL)
        c = L.cfg
        y, idx, _ = oracle_lib.forward_tokens(L, range(c.T))
        _, _, sc = oracle_lib.route(L, want_scores=True)
        for t in range(c.T):
            G = scipy.special.softmax(sc[t].astype(np.float64))
            xr = L.x[t].astype(np.float64)
            dense = sum(G[i] * oracle_lib.expert(L, i, xr) for i in idx[t])
            if S:
                dense = dense + oracle_lib.expert(L, c.E, xr)
            np.testing.assert_allclose(y[t], dense, rtol=1e-12, atol=1e-14)


def test_unknown_gate_mode_rejected(oracle_lib):
    L = _with_gate(random_layer(24, T=3, d=8, h=8, E=4, k=2), 3)
    with pytest.raises(ValueError):
        oracle_lib.route(L)


# ---- noisy top-k gating, training form (Qiita summary, "Gating: Noisy Top-k
# Softmax"): H = clean + n * Softplus(x W_noise), G = softmax(KeepTopK(H, k)),
# and the smooth Load(X) ("Load-balancing losses"; estimator of Shazeer et
# al. 2017, appendix A) ----

def _noisy_identity(clean, nraw, noise, k, bias=None):
    """x = [clean | nraw], W_g = [I | 0], W_noise = [0 | I]: the clean and
    noise scores are exactly the given values."""
    clean = np.asarray(clean, np.float32)
    T, E = clean.shape
    x = np.concatenate([clean, np.asarray(nraw, np.float32)], 1)
    wg = np.concatenate([np.eye(E), np.zeros((E, E))], 1).astype(np.float32)
    L = layer(T, 2 * E, 4, E, k, x=x, w_gate=wg, b_gate=bias,
              w_up=np.zeros((E, 4, 2 * E)), w_down=np.zeros((E, 2 * E, 4)))
    L.w_noise = np.concatenate([np.zeros((E, E)), np.eye(E)], 1).astype(np.float32)
    return L, np.ascontiguousarray(noise, np.float32)


def _noisy_random(seed, T, E, k, d=24, bias=True):
    L = random_layer(seed, T=T, d=d, h=8, E=E, k=k, act=SWIGLU, bias=bias)
    rng = np.random.default_rng(seed + 100)
    L.w_noise = (rng.standard_normal((E, d)) * 0.3).astype(np.float32)
    return L, rng.standard_normal((T, E)).astype(np.float32)


def test_noisy_gate_with_zero_noise_is_the_inference_gate(oracle_lib):
    """n = 0 removes the noise term: the clean scores, kept experts and
    weights are exactly those of the deterministic router."""
    L, n = _noisy_random(41, T=30, E=8, k=2)
    r = oracle_lib.route_noisy(L, np.zeros_like(n))
    idx, w, sc = oracle_lib.route(L, want_scores=True)
    np.testing.assert_array_equal(r["clean"], sc)
    np.testing.assert_array_equal(r["h"], sc)
    np.testing.assert_array_equal(r["idx"], idx)
    np.testing.assert_array_equal(r["w"], w)


def test_noise_scale_is_softplus(oracle_lib):
    """Scale = Softplus(x W_noise) = log(1 + e^v) (numpy logaddexp) rounded
    to float32; W_noise = 0 gives ln 2; a very negative v gives 0."""
    L, n = _noisy_random(42, T=40, E=6, k=2)
    r = oracle_lib.route_noisy(L, n)
    Ln = random_layer(42, T=40, d=24, h=8, E=6, k=2, act=SWIGLU)
    Ln.w_gate = L.w_noise
    _, _, nraw = oracle_lib.route(Ln, want_scores=True)
    ref = np.logaddexp(0.0, nraw.astype(np.float64)).astype(np.float32)
    np.testing.assert_allclose(r["scale"], ref, rtol=1.2e-7, atol=0)
    L0, n0 = _noisy_identity([[1.0, 2.0, -3.0]], [[0.0, -200.0, 50.0]], [[1.0, 1.0, 1.0]], 1)
    s = oracle_lib.route_noisy(L0, n0)["scale"][0]
    assert s[0] == np.float32(math.log(2.0)) and s[1] == 0.0 and s[2] == np.float32(50.0)


def _round_f32(q):
    """The float32 nearest to the rational q (ties to even)."""
    from fractions import Fraction
    c = np.float32(float(q))
    best = None
    for v in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        dist = abs(Fraction(float(v)) - q)
        if best is None or dist < best[0] or (dist == best[0] and int(v.view(np.uint32)) % 2 == 0):
            best = (dist, v)
    return best[1]


def test_noisy_scores_are_one_fused_multiply_add(oracle_lib):
    """H = clean + n * scale with a single rounding (exact rational sum
    rounded to the nearest float32)."""
    from fractions import Fraction
    L, n = _noisy_random(43, T=50, E=8, k=2)
    r = oracle_lib.route_noisy(L, n)
    for t in range(50):
        for e in range(8):
            q = Fraction(float(r["clean"][t, e])) + Fraction(float(n[t, e])) * Fraction(float(r["scale"][t, e]))
            assert r["h"][t, e] == _round_f32(q), (t, e)


@pytest.mark.parametrize("k", [1, 2, 5])
def test_noisy_topk_and_kept_softmax(oracle_lib, k):
    """Kept experts = stable descending order of H (numpy), weights = scipy
    softmax over the kept H."""
    L, n = _noisy_random(44 + k, T=60, E=8, k=k)
    r = oracle_lib.route_noisy(L, n)
    order = np.argsort(-r["h"].astype(np.float64), axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(r["idx"], order)
    ref = scipy.special.softmax(np.take_along_axis(r["h"], order, 1).astype(np.float64), axis=1)
    np.testing.assert_allclose(r["w"], ref, rtol=1e-13, atol=0)


def test_smooth_load_two_experts_closed_form(oracle_lib):
    """E = 2, k = 1: expert 0 stays chosen while its noisy score beats H_1,
    so P(x, 0) = Phi((clean_0 - H_1) / scale_0), and symmetrically."""
    rng = np.random.default_rng(45)
    clean = rng.standard_normal((20, 2)).astype(np.float32)
    nraw = rng.standard_normal((20, 2)).astype(np.float32)
    noise = rng.standard_normal((20, 2)).astype(np.float32)
    L, n = _noisy_identity(clean, nraw, noise, 1)
    r = oracle_lib.route_noisy(L, n)
    h, s = r["h"].astype(np.float64), r["scale"].astype(np.float64)
    c = clean.astype(np.float64)
    np.testing.assert_allclose(r["p"][:, 0], scipy.stats.norm.cdf((c[:, 0] - h[:, 1]) / s[:, 0]),
                               rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(r["p"][:, 1], scipy.stats.norm.cdf((c[:, 1] - h[:, 0]) / s[:, 1]),
                               rtol=1e-12, atol=1e-300)


def test_smooth_load_is_the_probability_of_staying_in_the_top_k(oracle_lib):
    """Brute force: redraw expert i's noise 200000 times with the other
    noisy scores fixed and count how often i is among the first k of a
    stable descending order; P(x, i) agrees within the Monte Carlo error."""
    L, n = _noisy_random(46, T=4, E=6, k=2)
    r = oracle_lib.route_noisy(L, n)
    rng = np.random.default_rng(47)
    draws = rng.standard_normal(200000)
    for t in range(4):
        h = r["h"][t].astype(np.float64)
        for i in range(6):
            hi = r["clean"][t, i] + draws * float(r["scale"][t, i])
            others = np.delete(np.arange(6), i)
            ahead = np.zeros(draws.size, np.int64)
            for j in others:
                ahead += (h[j] > hi) | ((h[j] == hi) & (j < i))
            p_mc = float(np.mean(ahead < 2))
            p = float(r["p"][t, i])
            assert abs(p - p_mc) <= 5 * math.sqrt(max(p * (1 - p), 1e-6) / draws.size) + 1e-4, (t, i, p, p_mc)


def test_smooth_load_edge_cases(oracle_lib):
    """k = E: every expert always stays (P = 1).  A zero noise scale makes P
    the indicator of clean score > threshold."""
    L, n = _noisy_random(48, T=10, E=4, k=4)
    assert np.all(oracle_lib.route_noisy(L, n)["p"] == 1.0)
    clean = [[3.0, 2.0, 1.0, 0.0]]
    L, n = _noisy_identity(clean, [[-200.0] * 4], [[1.0] * 4], 2)
    r = oracle_lib.route_noisy(L, n)
    assert r["scale"].max() == 0.0 and r["idx"][0].tolist() == [0, 1]
    # kept 0, 1: thresholds H_2 = 1 (excluding a kept one); unkept: H_1 = 2
    assert r["p"][0].tolist() == [1.0, 1.0, 0.0, 0.0]


def test_smooth_load_and_importance_sums(oracle_lib):
    """Load = column sums of P, Importance = sums of the kept weights; with
    k = E Load is T for every expert (CV^2 0)."""
    L, n = _noisy_random(49, T=64, E=8, k=2)
    r = oracle_lib.route_noisy(L, n)
    cnt, imp = oracle_lib.counts(L.cfg, r["idx"], r["w"])
    assert cnt.sum() == 128 and imp.sum() == pytest.approx(64.0, rel=1e-12)
    load = r["p"].sum(0)
    assert np.all(load > 0) and np.all(load < 64)
    assert oracle_lib.cv2(np.full(8, 64.0)) == 0.0
    v = np.array([1.0, 3.0])
    assert oracle_lib.cv2(v) == pytest.approx(0.25, rel=1e-15)   # var 1, mean 2
