"""Backward pass of the MoE layer forward by automatic differentiation, in
float64 on the CPU with plain PyTorch ops.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check and the benchmark's CPU-baseline leg may use it.

What is differentiated (the layer of the "Sparsely-Gated MoE" Qiita
summary, section "Sparsely-Gated MoE layer formula", with the gate of
"Gating: Noisy Top-k Softmax" in its noise-free form):

    y(x) = sum_j G_j(x) E_{i_j}(x)  (+ the shared expert with weight 1)
    G    = softmax over the kept k of s = x W_g^T + b (the default gate; the
           bias-selects gate takes the softmax of x W_g^T over the kept k,
           the softmax-all gate the softmax over all E read at the kept k)
    loss = <dy, y> + w_imp * CV(Importance)^2 (+ w_load * CV(Load)^2)

where the kept experts i_j are the oracle's float32 top-k selection, held
fixed (the selection is a step function: its derivative is zero wherever it
exists, which is why the router learns only through the softmax weights,
techfeed summary, "The hardest part: making the router trainable").
Importance(X)_e = sum over tokens of the gate values of expert e, CV^2 its
squared coefficient of variation with the population variance (Qiita
summary, "Load-balancing losses").  With an expert capacity the dropped
slots contribute nothing to y (their gate still counts in Importance, the
router's view).  Expert FFNs: Linear -> exact GELU -> Linear with biases,
or SwiGLU silu(x W1^T) * (x W3^T) -> W2 with W1 and W3 packed as [2h, d]
("Understanding MoE in Transformers", "Weight Loading Refactor").

The noisy gate (Qiita summary, "Gating: Noisy Top-k Softmax", training
form): H = s + n * Softplus(x W_noise^T) with the draws n given; G = the
softmax of H over the kept k; the smooth Load_i = sum over tokens of
Phi((s_i - kth_i) / Softplus_i), kth_i the k-th largest H without entry i
(Shazeer et al.'s estimator, "Load-balancing losses").  The kept experts
and the entry behind each kth_i come from the C oracle's float32 order of
H and are held fixed, like the selection.
Everything is evaluated in float64 from the exact values of the stored
float32 / bfloat16 numbers; torch.autograd does the differentiation.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import route as _route
from . import route_noisy as _route_noisy

NAMES = ("x", "w_gate", "b_gate", "w_up", "w_down", "b_up", "b_down",
         "w_up_shared", "w_down_shared", "w_noise")


def _f64(a) -> Optional[torch.Tensor]:
    """Exact float64 values of a float32 array or of bfloat16 bit patterns."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return torch.from_numpy(np.ascontiguousarray(a, np.float64))


def params(layer) -> dict:
    """Leaf float64 tensors (requires_grad) of every array the layer has."""
    out = {}
    for n in NAMES:
        t = _f64(getattr(layer, n, None))
        if t is not None and t.numel() > 0:
            out[n] = t.requires_grad_(True)
    return out


def _ffn(cfg, p, e: int, xr: torch.Tensor) -> torch.Tensor:
    """Expert e (e == E: the shared expert) on the rows xr."""
    shared = e == cfg.E
    w1 = p["w_up_shared"][0] if shared else p["w_up"][e]
    w2 = p["w_down_shared"][0] if shared else p["w_down"][e]
    if cfg.act == 0:   # GELU
        a = xr @ w1.T
        if "b_up" in p and not shared:
            a = a + p["b_up"][e]
        hid = 0.5 * a * (1.0 + torch.special.erf(a / np.sqrt(2.0)))
        out = hid @ w2.T
        if "b_down" in p and not shared:
            out = out + p["b_down"][e]
        return out
    h = cfg.h
    g = xr @ w1[:h].T
    u = xr @ w1[h:].T
    return (g * torch.sigmoid(g) * u) @ w2.T


def preactivations(layer, e: int, xrows: np.ndarray) -> np.ndarray:
    """Pre-activations of expert e (e == E: the shared one) on float rows:
    SwiGLU [x W1^T | x W3^T] (gate rows, then up rows), GELU x W1^T + b1;
    float64 [n, N_up]."""
    cfg = layer.cfg
    p = {n: t.detach() for n, t in params(layer).items()}
    shared = e == cfg.E
    w1 = p["w_up_shared"][0] if shared else p["w_up"][e]
    a = torch.from_numpy(np.asarray(xrows, np.float64)) @ w1.T
    if cfg.act == 0 and "b_up" in p and not shared:
        a = a + p["b_up"][e]
    return a.numpy()


def noisy_selection(layer, noise: np.ndarray):
    """The C oracle's float32 noisy selection: (idx [T, k], kth [T, E] or
    None when k = E), kth[t, e] the entry of H behind the threshold of e: the
    (k+1)-th of the stable descending order when e is kept, else the k-th."""
    cfg = layer.cfg
    r = _route_noisy(layer, noise)
    order = np.argsort(-r["h"].astype(np.float64), axis=1, kind="stable")
    assert np.array_equal(order[:, : cfg.k], r["idx"])
    if cfg.k == cfg.E:
        return r["idx"], None
    kept = np.zeros((cfg.T, cfg.E), bool)
    np.put_along_axis(kept, r["idx"].astype(np.int64), True, axis=1)
    kth = np.where(kept, order[:, cfg.k : cfg.k + 1], order[:, cfg.k - 1 : cfg.k])
    return r["idx"], kth


def _noisy_scores(p: dict, s: torch.Tensor, noise: torch.Tensor):
    """(H, Softplus of the noise scores) in float64."""
    u = p["x"] @ p["w_noise"].T
    sig = torch.nn.functional.softplus(u, beta=1.0, threshold=50.0)
    return s + noise * sig, sig


def _gates(layer, p: dict, idx: np.ndarray, noisy: Optional[dict] = None):
    """(gate values [T, k], Importance [E], smooth Load [E] or None) of the
    fixed selection idx, float64, from x and the router weights in p."""
    cfg = layer.cfg
    T, E = p["x"].shape[0], cfg.E
    raw = p["x"] @ p["w_gate"].T
    s = raw + p["b_gate"] if "b_gate" in p else raw
    it = torch.from_numpy(np.ascontiguousarray(idx, np.int64))
    gate = getattr(cfg, "gate", 0)
    load = None
    if noisy is not None:   # softmax over the kept noisy scores; smooth Load
        H, sig = _noisy_scores(p, s, _f64(noisy["noise"]))
        g = torch.softmax(torch.gather(H, 1, it), dim=1)
        if noisy["kth"] is None:   # k = E: every P is 1
            load = torch.full((E,), float(T), dtype=torch.float64)
        else:
            thr = torch.gather(H, 1, torch.from_numpy(np.ascontiguousarray(noisy["kth"],
                                                                           np.int64)))
            z = (s - thr) / sig
            load = (0.5 * torch.special.erfc(-z / np.sqrt(2.0))).sum(0)
    elif gate == 1:   # the bias steers the selection only
        g = torch.softmax(torch.gather(raw, 1, it), dim=1)
    elif gate == 2:   # softmax over all E, read at the kept experts
        g = torch.gather(torch.softmax(s, dim=1), 1, it)
    else:             # softmax over the kept k
        g = torch.softmax(torch.gather(s, 1, it), dim=1)
    imp = torch.zeros(E, dtype=torch.float64).index_add(0, it.reshape(-1), g.reshape(-1))
    return g, imp, load


def forward(layer, p: dict, idx: np.ndarray, keep: Optional[np.ndarray] = None,
            assign: Optional[np.ndarray] = None, noisy: Optional[dict] = None):
    """(y [T, d], gate values [T, k], Importance [E], Load [E] or None) as
    float64 tensors for the fixed selection idx [T, k]; assign [T*k]
    (next-choice re-routing): the expert that computes each slot, -1
    dropped, the gate values still those of idx; noisy: dict(noise [T, E],
    kth [T, E] or None) for the noisy gate."""
    cfg = layer.cfg
    T, k, E = cfg.T, cfg.k, cfg.E
    x = p["x"]
    g, imp, load = _gates(layer, p, idx, noisy)
    gk = g
    if keep is not None:
        gk = g * torch.from_numpy(np.asarray(keep, np.float64).reshape(T, k))
    y = torch.zeros((T, cfg.d), dtype=torch.float64)
    by = idx if assign is None else np.asarray(assign).reshape(T, k)
    for e in range(E):
        t_sel, j_sel = np.nonzero(by == e)
        if t_sel.size == 0:
            continue
        ts = torch.from_numpy(t_sel)
        out = _ffn(cfg, p, e, x[ts])
        y = y.index_add(0, ts, gk[ts, torch.from_numpy(j_sel)].unsqueeze(1) * out)
    if cfg.S:
        y = y + _ffn(cfg, p, E, x)
    return y, g, imp, load


def cv2(v: torch.Tensor) -> torch.Tensor:
    m = v.mean()
    if float(m.detach()) == 0.0:
        return torch.zeros((), dtype=v.dtype)
    return ((v - m) ** 2).mean() / (m * m)


def loss(layer, p: dict, idx, dy: torch.Tensor, keep=None, importance_weight: float = 0.0,
         assign=None, noisy=None, load_weight: float = 0.0):
    y, _, imp, load = forward(layer, p, idx, keep, assign, noisy)
    L = (dy * y).sum()
    if importance_weight:
        L = L + importance_weight * cv2(imp)
    if load_weight and load is not None:
        L = L + load_weight * cv2(load)
    return L


def backward(layer, dy: np.ndarray, keep: Optional[np.ndarray] = None,
             importance_weight: float = 0.0, idx: Optional[np.ndarray] = None,
             assign: Optional[np.ndarray] = None, noise: Optional[np.ndarray] = None,
             load_weight: float = 0.0) -> dict:
    """Gradients (float64 numpy, keyed by the array names, 'x' included) of
    <dy, y> + importance_weight * CV^2(Importance) with the oracle's routing
    (or the given selection idx; assign: the computing expert of each slot
    under next-choice re-routing).  noise [T, E]: the noisy gate with these
    draws (its selection from the C oracle), plus load_weight * CV^2(Load)."""
    noisy = None
    if noise is not None:
        idx, kth = noisy_selection(layer, noise)
        noisy = dict(noise=np.asarray(noise, np.float32), kth=kth)
    elif idx is None:
        idx, _, _ = _route(layer)
    p = params(layer)
    L = loss(layer, p, idx, _f64(dy), keep, importance_weight, assign, noisy, load_weight)
    names = list(p)
    grads = torch.autograd.grad(L, [p[n] for n in names], allow_unused=True)
    return {n: (np.zeros(tuple(p[n].shape)) if g is None else g.numpy())
            for n, g in zip(names, grads)}


# ---- slices of the same gradient for layers too large for the whole graph.
# Both follow from the loss by separability, and both are pinned to
# backward() on small layers: a token's x enters the loss only through its
# own output row and its own gate values in Importance (so with the
# Importance term replaced by its linearisation at the whole batch, the
# loss of a token subset has the same gradient in those tokens' x); and the
# expert FFN is a sum over hidden units (so the loss restricted to some
# hidden units of one expert has the same gradient in those units' weights).

def _router_params(layer) -> dict:
    """x, w_gate (and b_gate, w_noise) as float64 tensors, no expert weights."""
    p = {"x": _f64(layer.x), "w_gate": _f64(layer.w_gate)}
    for n in ("b_gate", "w_noise"):
        if getattr(layer, n, None) is not None:
            p[n] = _f64(getattr(layer, n))
    return p


def balance_gradients(layer, importance_weight: float, idx=None, noisy=None,
                      load_weight: float = 0.0):
    """d (w_imp CV^2(Importance) + w_load CV^2(Load)) / d (Importance, Load)
    at the whole batch, float64 [E] each (the oracle's routing unless idx is
    given; noisy: dict(noise, kth) of the noisy gate)."""
    if idx is None:
        idx, _, _ = _route(layer)
    _, imp, load = _gates(layer, _router_params(layer), idx, noisy)
    imp = imp.detach().requires_grad_(True)
    (gi,) = torch.autograd.grad(importance_weight * cv2(imp), [imp])
    gl = torch.zeros_like(imp)
    if load is not None and load_weight:
        load = load.detach().requires_grad_(True)
        (gl,) = torch.autograd.grad(load_weight * cv2(load), [load])
    return gi.numpy(), gl.numpy()


class _TokenSubset:
    """The layer restricted to some tokens (same weights, T = len(tokens))."""

    def __init__(self, layer, tokens):
        self.cfg = layer.cfg.with_(T=len(tokens))
        self.x = np.ascontiguousarray(np.asarray(layer.x)[np.asarray(tokens)])


def dx_rows(layer, dy: np.ndarray, tokens, importance_weight: float = 0.0,
            idx: Optional[np.ndarray] = None, noise: Optional[np.ndarray] = None,
            load_weight: float = 0.0, selection=None) -> np.ndarray:
    """Rows `tokens` of d loss / d x (loss of backward(), no capacity),
    float64 [len(tokens), d]; the balance terms are linearised at the whole
    batch.  noise: the noisy gate with these draws (selection: its
    noisy_selection(), computed if None).  Only the experts those tokens use
    are taken to float64."""
    tokens = np.asarray(tokens, np.int64)
    noisy = noisy_sub = None
    if noise is not None:
        idx, kth = selection if selection is not None else noisy_selection(layer, noise)
        noisy = dict(noise=np.asarray(noise, np.float32), kth=kth)
        noisy_sub = dict(noise=noisy["noise"][tokens], kth=None if kth is None else kth[tokens])
    elif idx is None:
        idx, _, _ = _route(layer)
    gi, gl = balance_gradients(layer, importance_weight, idx, noisy, load_weight)
    gimp, gload = torch.from_numpy(gi), torch.from_numpy(gl)
    sub = _TokenSubset(layer, tokens)
    p = _router_params(layer)
    p["x"] = _f64(sub.x).requires_grad_(True)
    used = sorted(set(np.asarray(idx)[tokens].ravel().tolist()))
    for n in ("w_up", "w_down", "b_up", "b_down"):
        a = getattr(layer, n, None)
        if a is not None and np.asarray(a).size:
            p[n] = {e: _f64(np.asarray(a)[e]) for e in used}
    for n in ("w_up_shared", "w_down_shared"):
        a = getattr(layer, n, None)
        if a is not None and np.asarray(a).size:
            p[n] = _f64(a)
    y, _, imp, load = forward(sub, p, idx[tokens], noisy=noisy_sub)
    L = (_f64(np.asarray(dy)[tokens]) * y).sum() + (gimp * imp).sum()
    if load is not None:
        L = L + (gload * load).sum()
    (gx,) = torch.autograd.grad(L, [p["x"]])
    return gx.numpy()


def expert_unit_grads(layer, dy: np.ndarray, e: int, units, idx: Optional[np.ndarray] = None,
                      w: Optional[np.ndarray] = None, noise: Optional[np.ndarray] = None,
                      selection=None) -> dict:
    """Gradients of the loss of backward() (no capacity) in the weights of
    hidden units `units` of expert e (e == E: the shared expert), float64:
    'w_up' [len(units), d] (SwiGLU: [2, len(units), d], gate rows then up
    rows), 'w_down' [d, len(units)], and 'b_up' [len(units)] for a GELU
    expert with biases.  The expert's rows: every slot routed to it with its
    gate value (the shared expert: every token, weight 1).  idx: the
    selection (the oracle's routing if None); w: its gate values [T, k]
    (those of forward()'s graph if None); noise: the noisy gate with these
    draws (selection: its noisy_selection(), computed if None)."""
    cfg = layer.cfg
    units = np.asarray(units, np.int64)
    xs = _f64(layer.x)
    dyt = _f64(np.asarray(dy))
    if e == cfg.E:
        rows_t = np.arange(cfg.T)
        gw = torch.ones(cfg.T, dtype=torch.float64)
        w1 = _f64(layer.w_up_shared)[0]
        w2 = _f64(layer.w_down_shared)[0]
        b1 = None
    else:
        noisy = None
        if noise is not None:
            idx, kth = selection if selection is not None else noisy_selection(layer, noise)
            noisy = dict(noise=np.asarray(noise, np.float32), kth=kth)
        elif idx is None:
            idx, _, _ = _route(layer)
        if w is None:   # the gate values of backward()'s graph
            w = _gates(layer, _router_params(layer), idx, noisy)[0].numpy()
        t_sel, j_sel = np.nonzero(idx == e)
        rows_t = t_sel
        gw = torch.from_numpy(np.asarray(w, np.float64)[t_sel, j_sel])
        w1 = _f64(np.asarray(layer.w_up)[e])
        w2 = _f64(np.asarray(layer.w_down)[e])
        b1 = (_f64(np.asarray(layer.b_up)[e])
              if getattr(layer, "b_up", None) is not None and np.asarray(layer.b_up).size
              else None)
    h = cfg.h
    xr = xs[torch.from_numpy(rows_t)]
    dyr = dyt[torch.from_numpy(rows_t)] * gw.unsqueeze(1)
    if cfg.act == 0:   # GELU
        w1u = w1[torch.from_numpy(units)].clone().requires_grad_(True)
        b1u = b1[torch.from_numpy(units)].clone().requires_grad_(True) if b1 is not None else None
        a = xr @ w1u.T + (b1u if b1u is not None else 0.0)
        hid = 0.5 * a * (1.0 + torch.special.erf(a / np.sqrt(2.0)))
        leaves = [w1u] + ([b1u] if b1u is not None else [])
    else:
        w1u = torch.stack([w1[torch.from_numpy(units)], w1[torch.from_numpy(units + h)]])
        w1u = w1u.clone().requires_grad_(True)
        g = xr @ w1u[0].T
        u = xr @ w1u[1].T
        hid = g * torch.sigmoid(g) * u
        leaves = [w1u]
    w2u = w2[:, torch.from_numpy(units)].clone().requires_grad_(True)
    L = (dyr * (hid @ w2u.T)).sum()
    grads = torch.autograd.grad(L, leaves + [w2u])
    out = {"w_up": grads[0].numpy(), "w_down": grads[-1].numpy()}
    if cfg.act == 0 and b1 is not None:
        out["b_up"] = grads[1].numpy()
    return out


# ---- the router's weight gradients at sizes too large for the whole graph.
# The router parameters (W_g, b_g, W_noise) enter the loss only through the
# gate values: the expert outputs and the shared expert do not depend on
# them.  So with every slot's expert output E_{i_j}(x_t) held fixed, the
# loss restricted to the router,
#     sum_t sum_j G_tj <dy_t, E_{i_j}(x_t)> + w_imp CV^2(Importance)
#                                          (+ w_load CV^2(Load)),
# has the same gradient in those parameters as the whole loss of backward()
# (pinned to it on small layers).

def slot_dy_products(layer, dy: np.ndarray, experts: np.ndarray, chunk: int = 256) -> np.ndarray:
    """c[t, j] = <dy_t, E_e(x_t)> with e = experts[t, j] (the computing
    expert of the slot, -1 for a dropped one: 0), float64 [T, k], from the C
    oracle's float64 expert outputs, a chunk of tokens at a time."""
    from . import slot_outputs as _slot_outputs
    cfg = layer.cfg
    dyf = np.asarray(dy, np.float64)
    out = np.empty((cfg.T, cfg.k), np.float64)
    for t0 in range(0, cfg.T, chunk):
        toks = np.arange(t0, min(cfg.T, t0 + chunk))
        ys = _slot_outputs(layer, toks, experts)
        out[toks] = np.einsum("tjd,td->tj", ys, dyf[toks])
    return out


def router_grads(layer, slot_dy: np.ndarray, importance_weight: float = 0.0,
                 idx: Optional[np.ndarray] = None, noise: Optional[np.ndarray] = None,
                 load_weight: float = 0.0, selection=None) -> dict:
    """Gradients of the loss of backward() in w_gate, b_gate and w_noise
    (those the layer has), float64, from slot_dy = slot_dy_products(...) for
    the same selection: idx (the oracle's routing if None), or the noisy
    gate with these draws (selection: its noisy_selection(), computed if
    None)."""
    noisy = None
    if noise is not None:
        idx, kth = selection if selection is not None else noisy_selection(layer, noise)
        noisy = dict(noise=np.asarray(noise, np.float32), kth=kth)
    elif idx is None:
        idx, _, _ = _route(layer)
    p = _router_params(layer)
    leaves = [n for n in ("w_gate", "b_gate", "w_noise") if n in p]
    for n in leaves:
        p[n].requires_grad_(True)
    g, imp, load = _gates(layer, p, idx, noisy)
    L = (g * torch.from_numpy(np.asarray(slot_dy, np.float64))).sum()
    if importance_weight:
        L = L + importance_weight * cv2(imp)
    if load_weight and load is not None:
        L = L + load_weight * cv2(load)
    grads = torch.autograd.grad(L, [p[n] for n in leaves], allow_unused=True)
    return {n: (np.zeros(tuple(p[n].shape)) if gr is None else gr.numpy())
            for n, gr in zip(leaves, grads)}
