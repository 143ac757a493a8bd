"""Seeded synthetic inputs for the MoE layer forward.

Both the HIP path and the CPU oracle are fed from here; this module holds
none of the method's arithmetic (no routing, no expert FFN, no combine).

Recipe (one numpy ``SeedSequence(seed)`` spawned into independent streams,
so any expert can be regenerated alone and experts are drawn in parallel):

  child 0       x [T, d] ~ N(0, 1) float32; for the GPT-2 layer each row is
                LayerNorm'd (eps 1e-5, no affine, float32) first
  child 1       W_g [E, d] ~ N(0, 0.02) float32 (the router stays fp32)
  child 2       b_g [E]: "normal0.5" -> N(0, 0.5); "zipf1.1" -> ln p_e with
                p_e proportional to (e + 1)^-1.1 (no draw); "none" -> absent
  child 3 + e   expert e: W_up[e] [N_up, d] then W_down[e] [d, h] ~ N(0, 0.02)
  child 3 + E   shared expert: W_up_s [2h, d] then W_down_s [d, h]

Noisy gating (training-time routing) draws from SeedSequence([seed, 1]),
spawned into two streams: W_noise [E, d] ~ N(0, 0.02) float32, then the
standard-normal noise [T, E] float32 (``make_noisy_gate``).

Every draw is float32; bf16 layers round each value to bfloat16 with
round-to-nearest-even and store the 16-bit patterns as ``uint16``.
GELU experts of the tiny layer carry zero-filled biases b1 [E, h], b2 [E, d].
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import BF16, F32, LayerConfig

WEIGHT_STD = 0.02


def f32_to_bf16_bits(a: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("synthetic draws must be finite")
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    if out is None:
        return r.astype(np.uint16)
    out[...] = r.reshape(out.shape)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray                 # [T, d]  float32 or uint16 (bf16 bits)
    w_gate: np.ndarray            # [E, d]  float32
    b_gate: Optional[np.ndarray]  # [E]     float32 or None
    w_up: np.ndarray              # [E, N_up, d]
    w_down: np.ndarray            # [E, d, h]
    b_up: Optional[np.ndarray]    # [E, h]  (GELU only) or None
    b_down: Optional[np.ndarray]  # [E, d]  (GELU only) or None
    w_up_shared: Optional[np.ndarray]    # [S, 2h, d] or None
    w_down_shared: Optional[np.ndarray]  # [S, d, h] or None

    def to_f32(self, a: Optional[np.ndarray]) -> Optional[np.ndarray]:
        if a is None:
            return None
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def _store_dtype(cfg: LayerConfig):
    return np.uint16 if cfg.dtype == BF16 else np.float32


def _fill(cfg: LayerConfig, dst: np.ndarray, vals: np.ndarray) -> None:
    if cfg.dtype == BF16:
        f32_to_bf16_bits(vals, out=dst)
    else:
        dst[...] = vals


def _draw_expert(cfg: LayerConfig, seq: np.random.SeedSequence,
                 up_dst: np.ndarray, down_dst: np.ndarray) -> None:
    rng = np.random.Generator(np.random.PCG64(seq))
    up = rng.standard_normal(up_dst.shape, dtype=np.float32)
    up *= np.float32(WEIGHT_STD)
    _fill(cfg, up_dst, up)
    del up
    down = rng.standard_normal(down_dst.shape, dtype=np.float32)
    down *= np.float32(WEIGHT_STD)
    _fill(cfg, down_dst, down)


def zipf_log_bias(E: int, s: float = 1.1) -> np.ndarray:
    """ln p_e for a Zipf(s) popularity over E experts, expert 0 most popular."""
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    return np.log(p).astype(np.float32)


def make_inputs(cfg: LayerConfig, workers: Optional[int] = None,
                experts: bool = True) -> LayerInputs:
    """Draw every input array of ``cfg`` from its seed (see module docstring).
    ``experts=False`` draws only x and the router (expert arrays are then
    zero-size placeholders); the drawn values do not change."""
    T, d, h, E = cfg.T, cfg.d, cfg.h, cfg.E
    children = np.random.SeedSequence(cfg.seed).spawn(3 + E + max(cfg.S, 1))

    rng_x = np.random.Generator(np.random.PCG64(children[0]))
    xf = rng_x.standard_normal((T, d), dtype=np.float32)
    if cfg.layernorm_x:
        mu = xf.mean(axis=1, keepdims=True, dtype=np.float32)
        var = ((xf - mu) ** 2).mean(axis=1, keepdims=True, dtype=np.float32)
        xf = ((xf - mu) / np.sqrt(var + np.float32(1e-5))).astype(np.float32)
    x = f32_to_bf16_bits(xf).reshape(T, d) if cfg.dtype == BF16 else xf

    rng_g = np.random.Generator(np.random.PCG64(children[1]))
    w_gate = rng_g.standard_normal((E, d), dtype=np.float32) * np.float32(WEIGHT_STD)

    if cfg.router_bias == "none":
        b_gate = None
    elif cfg.router_bias == "normal0.5":
        rng_b = np.random.Generator(np.random.PCG64(children[2]))
        b_gate = rng_b.standard_normal(E, dtype=np.float32) * np.float32(0.5)
    elif cfg.router_bias == "zipf1.1":
        b_gate = zipf_log_bias(E, 1.1)
    else:
        raise ValueError(cfg.router_bias)

    sd = _store_dtype(cfg)
    if not experts:
        empty = np.empty((0,), dtype=sd)
        return LayerInputs(cfg, x, w_gate, b_gate, empty, empty, None, None,
                           None, None)
    w_up = np.empty((E, cfg.n_up, d), dtype=sd)
    w_down = np.empty((E, d, h), dtype=sd)
    jobs = [(children[3 + e], w_up[e], w_down[e]) for e in range(E)]
    w_up_s = w_down_s = None
    if cfg.S:
        w_up_s = np.empty((cfg.S, 2 * h, d), dtype=sd)
        w_down_s = np.empty((cfg.S, d, h), dtype=sd)
        jobs.append((children[3 + E], w_up_s[0], w_down_s[0]))

    nw = workers or min(16, os.cpu_count() or 1)
    if nw <= 1 or len(jobs) == 1:
        for seq, u, dn in jobs:
            _draw_expert(cfg, seq, u, dn)
    else:
        with ThreadPoolExecutor(max_workers=nw) as ex:
            list(ex.map(lambda j: _draw_expert(cfg, *j), jobs))

    b_up = b_down = None
    if cfg.expert_bias and cfg.act == 0:
        b_up = np.zeros((E, h), dtype=sd)
        b_down = np.zeros((E, d), dtype=sd)

    return LayerInputs(cfg, x, w_gate, b_gate, w_up, w_down, b_up, b_down,
                       w_up_s, w_down_s)


def make_noisy_gate(cfg: LayerConfig):
    """(w_noise [E, d] float32, noise [T, E] float32) for noisy top-k gating
    of ``cfg``: the noise-scale router ~ N(0, 0.02) and the N(0, 1) draws."""
    a, b = np.random.SeedSequence([cfg.seed, 1]).spawn(2)
    w_noise = (np.random.Generator(np.random.PCG64(a))
               .standard_normal((cfg.E, cfg.d), dtype=np.float32) * np.float32(WEIGHT_STD))
    noise = np.random.Generator(np.random.PCG64(b)).standard_normal((cfg.T, cfg.E),
                                                                   dtype=np.float32)
    return w_noise, noise
