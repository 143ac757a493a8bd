"""Small hand-built layers for the tests (no arithmetic of the method)."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np

from synthetic import BF16, F32, GELU, SWIGLU, LayerConfig, f32_to_bf16_bits


def layer(T, d, h, E, k, act=GELU, dtype=F32, S=0, *, x, w_gate, b_gate=None,
          w_up, w_down, b_up=None, b_down=None, w_up_shared=None,
          w_down_shared=None, gate=0):
    """Wrap hand-made float arrays as a layer; bf16 layers round them (RNE)."""
    cfg = LayerConfig("hand", T=T, d=d, h=h, E=E, k=k, act=act, dtype=dtype, S=S,
                      gate=gate)

    def q(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a, np.float32)
        return f32_to_bf16_bits(a).reshape(a.shape) if dtype == BF16 else a

    return SimpleNamespace(
        cfg=cfg, x=q(x),
        w_gate=np.ascontiguousarray(w_gate, np.float32),
        b_gate=None if b_gate is None else np.ascontiguousarray(b_gate, np.float32),
        w_up=q(w_up), w_down=q(w_down), b_up=q(b_up), b_down=q(b_down),
        w_up_shared=q(w_up_shared), w_down_shared=q(w_down_shared))


def random_layer(seed, T, d, h, E, k, act=GELU, dtype=F32, S=0, bias=False,
                 expert_bias=False, wstd=0.3, gate=0):
    rng = np.random.default_rng(seed)
    n_up = h if act == GELU else 2 * h
    return layer(
        T, d, h, E, k, act, dtype, S,
        x=rng.standard_normal((T, d)),
        w_gate=rng.standard_normal((E, d)) * wstd,
        b_gate=rng.standard_normal(E) * 0.5 if bias else None,
        w_up=rng.standard_normal((E, n_up, d)) * wstd,
        w_down=rng.standard_normal((E, d, h)) * wstd,
        b_up=rng.standard_normal((E, h)) * 0.1 if expert_bias else None,
        b_down=rng.standard_normal((E, d)) * 0.1 if expert_bias else None,
        w_up_shared=rng.standard_normal((1, 2 * h, d)) * wstd if S else None,
        w_down_shared=rng.standard_normal((1, d, h)) * wstd if S else None,
        gate=gate)


__all__ = ["layer", "random_layer", "BF16", "F32", "GELU", "SWIGLU"]
