"""Device-memory plumbing around the C ABI: upload a layer's arrays with
torch, allocate the outputs and the workspace once, and call the entry
points.  Torch only owns memory and streams here; all arithmetic of the
layer runs in libmoe.so."""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

from . import binding as B


def to_device(a: Optional[np.ndarray], device="cuda") -> Optional[torch.Tensor]:
    """numpy float32 -> float32 tensor; numpy uint16 (bf16 bits) -> bfloat16."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    raise TypeError(f"unsupported host dtype {a.dtype}")


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 device tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class DeviceLayer:
    """A layer's inputs resident in HBM, plus its C-ABI config and weights."""
    cfg: B.MoeConfig
    x: torch.Tensor
    w_gate: torch.Tensor
    b_gate: Optional[torch.Tensor]
    w_up: torch.Tensor
    w_down: torch.Tensor
    b_up: Optional[torch.Tensor]
    b_down: Optional[torch.Tensor]
    w_up_shared: Optional[torch.Tensor]
    w_down_shared: Optional[torch.Tensor]
    layout: int = B.MOE_LAYOUT_ROW_MAJOR

    @classmethod
    def upload(cls, layer, device="cuda", capacity: int = 0,
               overflow: int = 0) -> "DeviceLayer":
        """capacity: per-expert limit on kept assignments (0: no limit);
        overflow: what happens beyond it (0 drop, 1 next choice)."""
        return cls(B.config_of(layer.cfg, capacity, overflow), to_device(layer.x, device),
                   to_device(layer.w_gate, device), to_device(layer.b_gate, device),
                   to_device(layer.w_up, device), to_device(layer.w_down, device),
                   to_device(layer.b_up, device), to_device(layer.b_down, device),
                   to_device(layer.w_up_shared, device),
                   to_device(layer.w_down_shared, device))

    def weights(self) -> B.MoeWeights:
        return B.weights(self.w_gate, self.w_up, self.w_down, self.b_gate,
                         self.b_up, self.b_down, self.w_up_shared,
                         self.w_down_shared, self.layout)

    def tiled(self) -> "DeviceLayer":
        """The same layer with its four expert matrices rewritten by
        moe_tile_weights (bf16 layers; forward calls only)."""
        if self.layout == B.MOE_LAYOUT_TILED:
            return self

        def tile(w):
            if w is None:
                return None
            out = torch.empty_like(w)
            B.moe_tile_weights(w, out, 1, w.numel() // w.shape[-1], w.shape[-1])
            return out
        return replace(self, w_up=tile(self.w_up), w_down=tile(self.w_down),
                       w_up_shared=tile(self.w_up_shared),
                       w_down_shared=tile(self.w_down_shared),
                       layout=B.MOE_LAYOUT_TILED)

    @property
    def act_dtype(self):
        return torch.bfloat16 if self.cfg.dtype == B.MOE_DTYPE_BF16 else torch.float32


class Forward:
    """Preallocated outputs + workspace for repeated moe_forward calls."""

    def __init__(self, dl: DeviceLayer):
        c = dl.cfg
        dev = dl.x.device
        T, k, E, d = c.num_tokens, c.top_k, c.num_experts, c.d_model
        self.dl = dl
        self.w = dl.weights()
        self.y = torch.empty((T, d), dtype=dl.act_dtype, device=dev)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty((E,), dtype=torch.int32, device=dev)
        self.importance = torch.empty((E,), dtype=torch.float32, device=dev)
        self.stats = torch.empty((3,), dtype=torch.float64, device=dev)
        nb = B.moe_workspace_bytes(c)
        self.ws = torch.empty((max(nb, 256),), dtype=torch.uint8, device=dev)

    def __call__(self, stream=None) -> torch.Tensor:
        B.moe_forward(self.dl.cfg, self.w, self.dl.x, self.y, self.topk_idx,
                      self.topk_w, self.counts, self.importance, self.stats,
                      self.ws, stream=stream)
        return self.y
