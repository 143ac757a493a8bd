"""ctypes binding of libmoe.so (the C ABI declared in include/moe.h).

Argument marshalling only: every function has the name of its C entry
point, turns torch device tensors into raw device pointers and the current
torch stream into a hipStream_t, calls the library, and raises MoeError on
a non-OK status.  No step of the layer runs in Python; if libmoe.so is
missing, loading fails loudly (there is no fallback path).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_ACT_GELU = 0
MOE_ACT_SWIGLU = 1
MOE_GATE_TOPK_SOFTMAX = 0
MOE_GATE_BIAS_SELECTS = 1
MOE_GATE_SOFTMAX_ALL = 2
MOE_OVERFLOW_DROP = 0
MOE_OVERFLOW_NEXT_CHOICE = 1
MOE_LAYOUT_ROW_MAJOR = 0
MOE_LAYOUT_TILED = 1

# The ABI this binding marshals for (moe.h's MOE_ABI_VERSION): a library of
# another version may take other argument lists, so lib() refuses it.
ABI_VERSION = 10

EXPORTS = (
    "moe_abi_version", "moe_status_string", "moe_workspace_bytes",
    "moe_grouped_rows", "moe_route", "moe_permute", "moe_expert_up",
    "moe_expert_down", "moe_expert_ffn", "moe_combine", "moe_forward",
    "moe_param_counts", "moe_load_stats", "moe_expert_capacity",
    "moe_route_noisy", "moe_backward_workspace_bytes", "moe_backward",
    "moe_expert_up_train", "moe_permute_noalloc", "moe_tile_weights",
)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


class MoeConfig(C.Structure):
    _fields_ = [("num_tokens", C.c_int64), ("d_model", C.c_int32),
                ("d_hidden", C.c_int32), ("num_experts", C.c_int32),
                ("top_k", C.c_int32), ("num_shared", C.c_int32),
                ("act", C.c_int32), ("dtype", C.c_int32),
                ("capacity", C.c_int32), ("gate", C.c_int32),
                ("overflow", C.c_int32)]


class MoeWeights(C.Structure):
    _fields_ = [("w_gate", C.c_void_p), ("b_gate", C.c_void_p),
                ("w_up", C.c_void_p), ("b_up", C.c_void_p),
                ("w_down", C.c_void_p), ("b_down", C.c_void_p),
                ("w_up_shared", C.c_void_p), ("w_down_shared", C.c_void_p),
                ("layout", C.c_int32)]


_lib = None


def lib():
    """Load libmoe.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = C.CDLL(LIB_PATH)
        P, S = C.c_void_p, C.c_int
        L.moe_abi_version.restype = C.c_int
        L.moe_status_string.restype = C.c_char_p
        L.moe_status_string.argtypes = [S]
        sig = {
            "moe_workspace_bytes": [P, P],
            "moe_grouped_rows": [P, P],
            "moe_route": [P, P, P, P, P, P, P, P, P],
            "moe_backward_workspace_bytes": [P, P],
            "moe_backward": [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, C.c_float, P, P,
                             C.c_size_t, P],
            "moe_expert_up_train": [P, P, P, P, P, P, P, P, P],
            "moe_route_noisy": [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                C.c_size_t, P],
            "moe_permute": [P, P, P, P, P, P, P, P, P, P, P, P, P, C.c_size_t, P],
            "moe_permute_noalloc": [P, P, P, P, P, P, P, P, P, P, P, P, P],
            "moe_expert_up": [P, P, P, P, P, P, P, P],
            "moe_expert_down": [P, P, P, P, P, P],
            "moe_expert_ffn": [P, P, P, P, P, P, P, P, C.c_size_t, P],
            "moe_combine": [P, P, P, P, P, P],
            "moe_forward": [P, P, P, P, P, P, P, P, P, P, C.c_size_t, P],
            "moe_param_counts": [P, P, P],
            "moe_load_stats": [P, P, C.c_int32, P, P, P],
            "moe_expert_capacity": [C.c_int64, C.c_int32, C.c_int32, C.c_double, P],
            "moe_tile_weights": [P, P, C.c_int64, C.c_int32, C.c_int32, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = C.c_int
        got = L.moe_abi_version()
        if got != ABI_VERSION:
            raise RuntimeError(
                f"{LIB_PATH} implements ABI version {got}, this binding version "
                f"{ABI_VERSION}: rebuild it with __graft_entry__.build()")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_status_string(status: int) -> str:
    return status_string(status)


# ------------------------------------------------------------ marshalling --

def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or a raw int / None passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check(fn: str, st: int) -> None:
    if st != MOE_OK:
        raise MoeError(fn, st)


def config(T: int, d: int, h: int, E: int, k: int, act: int, dtype: int,
           S: int = 0, capacity: int = 0, gate: int = 0, overflow: int = 0) -> MoeConfig:
    return MoeConfig(int(T), int(d), int(h), int(E), int(k), int(S), int(act),
                     int(dtype), int(capacity), int(gate), int(overflow))


def config_of(c, capacity: int = 0, overflow: int = 0) -> MoeConfig:
    """From any object with T, d, h, E, k, S, act, dtype (and optionally
    gate) attributes."""
    return config(c.T, c.d, c.h, c.E, c.k, c.act, c.dtype, c.S, capacity,
                  getattr(c, "gate", 0), overflow)


def weights(w_gate, w_up, w_down, b_gate=None, b_up=None, b_down=None,
            w_up_shared=None, w_down_shared=None,
            layout: int = MOE_LAYOUT_ROW_MAJOR) -> MoeWeights:
    """Pointer struct; the caller keeps the tensors alive while it is used.
    layout: MOE_LAYOUT_TILED when the four expert matrices went through
    moe_tile_weights."""
    return MoeWeights(_ptr(w_gate), _ptr(b_gate), _ptr(w_up), _ptr(b_up),
                      _ptr(w_down), _ptr(b_down), _ptr(w_up_shared),
                      _ptr(w_down_shared), layout)


def moe_tile_weights(src, dst, count: int, rows: int, cols: int, stream=None) -> None:
    """dst (same size as src) = the count bf16 matrices [rows, cols] of src
    in the tiled order of MOE_LAYOUT_TILED."""
    _check("moe_tile_weights", lib().moe_tile_weights(
        _ptr(src), _ptr(dst), count, rows, cols, _stream(stream)))


# ------------------------------------------------------------ entry points --

def moe_workspace_bytes(cfg: MoeConfig) -> int:
    n = C.c_size_t()
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(C.byref(cfg), C.byref(n)))
    return n.value


def moe_grouped_rows(cfg: MoeConfig) -> int:
    n = C.c_int64()
    _check("moe_grouped_rows", lib().moe_grouped_rows(C.byref(cfg), C.byref(n)))
    return n.value


def moe_route(cfg, x, w_gate, b_gate, topk_idx, topk_w, counts, logits=None,
              stream=None) -> None:
    _check("moe_route", lib().moe_route(
        C.byref(cfg), _ptr(x), _ptr(w_gate), _ptr(b_gate), _ptr(topk_idx),
        _ptr(topk_w), _ptr(counts), _ptr(logits), _stream(stream)))


class MoeGrads(C.Structure):
    _fields_ = [("dx", C.c_void_p), ("dw_gate", C.c_void_p), ("db_gate", C.c_void_p),
                ("dw_up", C.c_void_p), ("dw_down", C.c_void_p), ("db_up", C.c_void_p),
                ("db_down", C.c_void_p), ("dw_up_shared", C.c_void_p),
                ("dw_down_shared", C.c_void_p)]


def grads(dx, dw_gate, dw_up, dw_down, db_gate=None, db_up=None, db_down=None,
          dw_up_shared=None, dw_down_shared=None) -> MoeGrads:
    return MoeGrads(_ptr(dx), _ptr(dw_gate), _ptr(db_gate), _ptr(dw_up), _ptr(dw_down),
                    _ptr(db_up), _ptr(db_down), _ptr(dw_up_shared), _ptr(dw_down_shared))


class MoeNoisyGrad(C.Structure):
    _fields_ = [("w_noise", C.c_void_p), ("noise", C.c_void_p),
                ("clean_logits", C.c_void_p), ("noise_scale", C.c_void_p),
                ("load", C.c_void_p), ("load_weight", C.c_float),
                ("dw_noise", C.c_void_p)]


def noisy_grad(w_noise, noise, clean_logits, noise_scale, dw_noise, load=None,
               load_weight: float = 0.0) -> MoeNoisyGrad:
    """Pointer struct of the noisy gate's backward inputs and W_noise output."""
    return MoeNoisyGrad(_ptr(w_noise), _ptr(noise), _ptr(clean_logits), _ptr(noise_scale),
                        _ptr(load), float(load_weight), _ptr(dw_noise))


def moe_backward_workspace_bytes(cfg: MoeConfig) -> int:
    n = C.c_size_t()
    _check("moe_backward_workspace_bytes",
           lib().moe_backward_workspace_bytes(C.byref(cfg), C.byref(n)))
    return n.value


def moe_backward(cfg, w: MoeWeights, x, dy, topk_idx, topk_w, offsets, pos, x_perm, y_perm,
                 importance, importance_weight: float, g: MoeGrads, ws, ws_bytes=None,
                 stream=None, hidden=None, preact=None, logits=None,
                 noisy: MoeNoisyGrad = None) -> None:
    nb = _nbytes(ws) if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check("moe_backward", lib().moe_backward(
        C.byref(cfg), C.byref(w), _ptr(x), _ptr(dy), _ptr(topk_idx), _ptr(topk_w),
        _ptr(offsets), _ptr(pos), _ptr(x_perm), _ptr(y_perm), _ptr(hidden), _ptr(preact),
        _ptr(logits), C.byref(noisy) if noisy is not None else None, _ptr(importance),
        float(importance_weight), C.byref(g), _ptr(ws), nb,
        _stream(stream)))


def moe_expert_up_train(cfg, w: MoeWeights, x_perm, x, offsets, hidden, preact,
                        stream=None, perm_src=None) -> None:
    """x_perm None: the token rows are x[perm_src[p]], read in place."""
    _check("moe_expert_up_train", lib().moe_expert_up_train(
        C.byref(cfg), C.byref(w), _ptr(x_perm), _ptr(perm_src), _ptr(x), _ptr(offsets),
        _ptr(hidden), _ptr(preact), _stream(stream)))


def moe_route_noisy(cfg, x, w_gate, b_gate, w_noise, noise, clean_logits, noise_scale,
                    topk_idx, topk_w, counts, importance, load, cv2, ws, ws_bytes=None,
                    stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check("moe_route_noisy", lib().moe_route_noisy(
        C.byref(cfg), _ptr(x), _ptr(w_gate), _ptr(b_gate), _ptr(w_noise), _ptr(noise),
        _ptr(clean_logits), _ptr(noise_scale), _ptr(topk_idx), _ptr(topk_w),
        _ptr(counts), _ptr(importance), _ptr(load), _ptr(cv2), _ptr(ws), nb,
        _stream(stream)))


def moe_permute(cfg, topk_idx, topk_w, x, offsets, perm_src, pos, importance,
                stats, x_perm, ws, ws_bytes=None, stream=None, logits=None,
                counts=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check("moe_permute", lib().moe_permute(
        C.byref(cfg), _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(x), _ptr(offsets),
        _ptr(perm_src), _ptr(pos), _ptr(importance), _ptr(stats), _ptr(counts), _ptr(x_perm),
        _ptr(ws), nb, _stream(stream)))


def moe_permute_noalloc(cfg, topk_idx, topk_w, x, offsets, perm_src, pos, importance,
                        stats, x_perm, stream=None, logits=None, counts=None) -> None:
    """moe_permute with the library's static scratch (no workspace)."""
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(
        C.byref(cfg), _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(x), _ptr(offsets),
        _ptr(perm_src), _ptr(pos), _ptr(importance), _ptr(stats), _ptr(counts), _ptr(x_perm),
        _stream(stream)))


def moe_expert_up(cfg, w: MoeWeights, x_perm, x, offsets, hidden,
                  stream=None, perm_src=None) -> None:
    """x_perm None: the token rows are x[perm_src[p]], read in place."""
    _check("moe_expert_up", lib().moe_expert_up(
        C.byref(cfg), C.byref(w), _ptr(x_perm), _ptr(perm_src), _ptr(x), _ptr(offsets),
        _ptr(hidden), _stream(stream)))


def moe_expert_down(cfg, w: MoeWeights, hidden, offsets, y_perm,
                    stream=None) -> None:
    _check("moe_expert_down", lib().moe_expert_down(
        C.byref(cfg), C.byref(w), _ptr(hidden), _ptr(offsets), _ptr(y_perm),
        _stream(stream)))


def moe_expert_ffn(cfg, w: MoeWeights, x_perm, x, offsets, y_perm, ws,
                   ws_bytes=None, stream=None, perm_src=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        C.byref(cfg), C.byref(w), _ptr(x_perm), _ptr(perm_src), _ptr(x), _ptr(offsets),
        _ptr(y_perm), _ptr(ws), nb, _stream(stream)))


def moe_combine(cfg, y_perm, pos, topk_w, y, stream=None) -> None:
    _check("moe_combine", lib().moe_combine(
        C.byref(cfg), _ptr(y_perm), _ptr(pos), _ptr(topk_w), _ptr(y),
        _stream(stream)))


def moe_forward(cfg, w: MoeWeights, x, y, topk_idx, topk_w, counts,
                importance, stats, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check("moe_forward", lib().moe_forward(
        C.byref(cfg), C.byref(w), _ptr(x), _ptr(y), _ptr(topk_idx),
        _ptr(topk_w), _ptr(counts), _ptr(importance), _ptr(stats), _ptr(ws),
        nb, _stream(stream)))


def moe_param_counts(cfg: MoeConfig):
    tot, act = C.c_int64(), C.c_int64()
    _check("moe_param_counts",
           lib().moe_param_counts(C.byref(cfg), C.byref(tot), C.byref(act)))
    return tot.value, act.value


def moe_expert_capacity(T: int, k: int, E: int, factor: float) -> int:
    cap = C.c_int32()
    _check("moe_expert_capacity",
           lib().moe_expert_capacity(int(T), int(k), int(E), float(factor), C.byref(cap)))
    return cap.value


def moe_load_stats(counts, importance=None):
    """Host arrays (numpy int32 counts, float32 importance or None)."""
    import numpy as np
    cnt = np.ascontiguousarray(counts, dtype=np.int32)
    imp = None if importance is None else np.ascontiguousarray(importance, dtype=np.float32)
    a, b, c = C.c_double(), C.c_double(), C.c_double()
    _check("moe_load_stats", lib().moe_load_stats(
        cnt.ctypes.data, None if imp is None else imp.ctypes.data, int(cnt.size),
        C.byref(a), C.byref(b), C.byref(c)))
    return a.value, b.value, c.value
