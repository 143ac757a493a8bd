"""The allocation-free dispatch (moe_permute_noalloc, the library's static
scratch) against moe_permute with a caller workspace, through the C ABI:
bit-exact grouping, row move, Importance, statistics and counts, on two
calls in a row, the second with a smaller batch (the static scratch keeps
the first call's contents)."""
import numpy as np
import pytest
import torch

from helpers import BF16, SWIGLU, random_layer
from sparse_mixture_experts_07_amd import binding as B
from sparse_mixture_experts_07_amd.device import DeviceLayer

pytestmark = pytest.mark.gpu


def _dispatch(L, capacity, overflow, noalloc):
    dl = DeviceLayer.upload(L, capacity=capacity, overflow=overflow)
    c, dev = dl.cfg, dl.x.device
    T, k, E, d = L.cfg.T, L.cfg.k, L.cfg.E, L.cfg.d
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    B.moe_route(c, dl.x, dl.w_gate, dl.b_gate, idx, w, None, logits)
    out = dict(offsets=torch.full((E + 1,), -5, dtype=torch.int32, device=dev),
               perm_src=torch.full((T * k,), -5, dtype=torch.int32, device=dev),
               pos=torch.full((T * k,), -5, dtype=torch.int32, device=dev),
               imp=torch.full((E,), -5.0, dtype=torch.float32, device=dev),
               stats=torch.full((3,), -5.0, dtype=torch.float64, device=dev),
               counts=torch.full((E,), -5, dtype=torch.int32, device=dev),
               x_perm=torch.zeros((T * k, d), dtype=torch.bfloat16, device=dev))
    args = (c, idx, w, dl.x, out["offsets"], out["perm_src"], out["pos"], out["imp"],
            out["stats"], out["x_perm"])
    if noalloc:
        B.moe_permute_noalloc(*args, logits=logits, counts=out["counts"])
    else:
        ws = torch.empty(B.moe_workspace_bytes(c), dtype=torch.uint8, device=dev)
        B.moe_permute(*args, ws, logits=logits, counts=out["counts"])
    torch.cuda.synchronize()
    n = int(out["offsets"][E].item())
    return {key: (v[:n] if key in ("perm_src", "x_perm") else v).cpu() for key, v in out.items()}


@pytest.mark.parametrize("capacity,overflow", [(0, 0), (400, 0), (400, B.MOE_OVERFLOW_NEXT_CHOICE)],
                         ids=["no-capacity", "drop", "next-choice"])
def test_noalloc_dispatch_equals_workspace_dispatch(capacity, overflow):
    # the first batch takes the multi-workgroup grouping (18000 assignments),
    # the second the single-workgroup one (1800)
    for T in (3000, 300):
        L = random_layer(T, T=T, d=128, h=64, E=64, k=6, act=SWIGLU, dtype=BF16, bias=True,
                         wstd=0.1)
        L.b_gate = np.linspace(1.0, -1.0, 64).astype(np.float32)
        cap = capacity if T == 3000 else capacity // 10
        ref = _dispatch(L, cap, overflow, noalloc=False)
        got = _dispatch(L, cap, overflow, noalloc=True)
        for key in ref:
            if ref[key].dtype == torch.bfloat16:
                assert torch.equal(ref[key].view(torch.int16), got[key].view(torch.int16)), key
            else:
                assert torch.equal(ref[key], got[key]), (T, key)
