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
    loss = <dy, y> + w_imp * CV(Importance)^2

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
Everything is evaluated in float64 from the exact values of the stored
float32 / bfloat16 numbers; torch.autograd does the differentiation.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import route as _route

NAMES = ("x", "w_gate", "b_gate", "w_up", "w_down", "b_up", "b_down",
         "w_up_shared", "w_down_shared")


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


def forward(layer, p: dict, idx: np.ndarray, keep: Optional[np.ndarray] = None,
            assign: Optional[np.ndarray] = None):
    """(y [T, d], gate values [T, k], Importance [E]) as float64 tensors for
    the fixed selection idx [T, k]; assign [T*k] (next-choice re-routing):
    the expert that computes each slot, -1 dropped, the gate values still
    those of idx."""
    cfg = layer.cfg
    T, k, E = cfg.T, cfg.k, cfg.E
    x = p["x"]
    raw = x @ p["w_gate"].T
    s = raw + p["b_gate"] if "b_gate" in p else raw
    it = torch.from_numpy(np.ascontiguousarray(idx, np.int64))
    gate = getattr(cfg, "gate", 0)
    if gate == 1:     # the bias steers the selection only
        g = torch.softmax(torch.gather(raw, 1, it), dim=1)
    elif gate == 2:   # softmax over all E, read at the kept experts
        g = torch.gather(torch.softmax(s, dim=1), 1, it)
    else:             # softmax over the kept k
        g = torch.softmax(torch.gather(s, 1, it), dim=1)
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
    imp = torch.zeros(E, dtype=torch.float64).index_add(0, it.reshape(-1), g.reshape(-1))
    return y, g, imp


def cv2(v: torch.Tensor) -> torch.Tensor:
    m = v.mean()
    if float(m.detach()) == 0.0:
        return torch.zeros((), dtype=v.dtype)
    return ((v - m) ** 2).mean() / (m * m)


def loss(layer, p: dict, idx, dy: torch.Tensor, keep=None, importance_weight: float = 0.0,
         assign=None):
    y, _, imp = forward(layer, p, idx, keep, assign)
    L = (dy * y).sum()
    if importance_weight:
        L = L + importance_weight * cv2(imp)
    return L


def backward(layer, dy: np.ndarray, keep: Optional[np.ndarray] = None,
             importance_weight: float = 0.0, idx: Optional[np.ndarray] = None,
             assign: Optional[np.ndarray] = None) -> dict:
    """Gradients (float64 numpy, keyed by the array names, 'x' included) of
    <dy, y> + importance_weight * CV^2(Importance) with the oracle's routing
    (or the given selection idx; assign: the computing expert of each slot
    under next-choice re-routing)."""
    if idx is None:
        idx, _, _ = _route(layer)
    p = params(layer)
    L = loss(layer, p, idx, _f64(dy), keep, importance_weight, assign)
    names = list(p)
    grads = torch.autograd.grad(L, [p[n] for n in names], allow_unused=True)
    return {n: (np.zeros(tuple(p[n].shape)) if g is None else g.numpy())
            for n, g in zip(names, grads)}
