"""LION layers of libgbla.so (C ABI in include/lion.h).

Bidirectional linear attention with a decay mask, from "Linear Attention for
Efficient Bidirectional Sequence Modeling" (method details: bidirectional mask
M = M^F + M^B - I, chunkwise form; the model table's Lion-s, Lion-d and
Lion-lit; feature map (SiLU + 0.5) / ||.||): q, k, v = x W, lambda =
sigmoid(x w_lam + b_lam) (decay "s"), sigmoid(b_lam) per head (decay "d") or 1
(decay "lit"), y = Scale((phi(Q) phi(K)^T) (.) M) V with row normalisation, per
packed sequence and head. `lion_forward` / `lion_backward` mirror the C entry points
(device pointers and the current HIP stream only); `forward` / `backward`
allocate outputs, cache and workspace. Every step runs in the HIP library.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import DTYPE_BF16, DTYPE_F32, LION_DECAY, LionProblem

__all__ = ["LionProblem", "problem", "workspace_size", "activation_size", "lion_forward", "lion_backward",
           "forward", "backward"]

CHUNK = 64


def _torch():
    import torch
    return torch


def problem(num_seqs: int, total_tokens: int, d_model: int, num_heads: int, head_dim: int, dtype,
            decay: str = "s") -> LionProblem:
    """Problem descriptor; dtype is a torch dtype or a DTYPE_* code; decay is
    "s" (Lion-s), "d" (Lion-d) or "lit" (Lion-lit)."""
    if isinstance(dtype, int):
        code = dtype
    else:
        torch = _torch()
        if dtype == torch.float32:
            code = DTYPE_F32
        elif dtype == torch.bfloat16:
            code = DTYPE_BF16
        else:
            raise TypeError(f"unsupported dtype {dtype}: float32 or bfloat16")
    return LionProblem(int(num_seqs), int(total_tokens), int(d_model), int(num_heads), int(head_dim), code, CHUNK,
                       LION_DECAY[decay])


def workspace_size(p: LionProblem, backward: bool) -> int:
    out = ctypes.c_size_t()
    _lib.check(_lib.load().lion_workspace_size(ctypes.byref(p), int(bool(backward)), ctypes.byref(out)),
               "lion_workspace_size")
    return out.value


def activation_size(p: LionProblem) -> int:
    out = ctypes.c_size_t()
    _lib.check(_lib.load().lion_activation_size(ctypes.byref(p), ctypes.byref(out)), "lion_activation_size")
    return out.value


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("all tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _nbytes(t):
    return ctypes.c_size_t(t.numel() * t.element_size())


def _check_common(p: LionProblem, x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam) -> None:
    """Sizes and dtypes of the arguments the forward and backward share, against p."""
    torch = _torch()
    dt = _lib._torch_dtype(p.dtype)
    T, d, H, D = p.total_tokens, p.d_model, p.num_heads, p.num_heads * p.head_dim
    _lib.need(x, "x", T * d, dt, required=T > 0)
    _lib.need(cu_seqlens, "cu_seqlens", p.num_seqs + 1, torch.int32)
    for name, w in (("w_q", w_q), ("w_k", w_k), ("w_v", w_v)):
        _lib.need(w, name, d * D, dt)
    _lib.need(w_lam, "w_lam", H * d, dt, required=False)
    _lib.need(b_lam, "b_lam", H, torch.float32, required=False)


def lion_forward(p: LionProblem, x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam, y, act, workspace, stream=None) -> None:
    """Enqueue the forward pass (include/lion.h: lion_forward); act may be None.
    Every tensor is checked against p (dtype, device, size) before anything is
    enqueued."""
    _check_common(p, x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam)
    _lib.need(y, "y", p.total_tokens * p.num_heads * p.head_dim, _lib._torch_dtype(p.dtype),
              required=p.total_tokens > 0)
    _lib.need_bytes(act, "act", activation_size(p), required=False)
    _lib.need_bytes(workspace, "workspace", 0)
    st = _lib.load().lion_forward(ctypes.byref(p), _ptr(x), _ptr(cu_seqlens), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                                  _ptr(w_lam), _ptr(b_lam), _ptr(y), _ptr(act), _ptr(workspace), _nbytes(workspace),
                                  _stream(stream))
    _lib.check(st, "lion_forward")


def lion_backward(p: LionProblem, x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam, act, y, dy, dx, dw_q, dw_k, dw_v,
                  dw_lam, db_lam, workspace, stream=None) -> None:
    """Enqueue the backward pass (include/lion.h: lion_backward). Every tensor
    is checked against p (dtype, device, size) before anything is enqueued."""
    torch = _torch()
    dt = _lib._torch_dtype(p.dtype)
    T, d, H, D = p.total_tokens, p.d_model, p.num_heads, p.num_heads * p.head_dim
    _check_common(p, x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam)
    _lib.need_bytes(act, "act", activation_size(p))
    _lib.need(y, "y", T * D, dt, required=T > 0)
    _lib.need(dy, "dy", T * D, dt, required=T > 0)
    _lib.need(dx, "dx", T * d, dt, required=T > 0)
    for name, t in (("dw_q", dw_q), ("dw_k", dw_k), ("dw_v", dw_v)):
        _lib.need(t, name, d * D, torch.float32)
    _lib.need(dw_lam, "dw_lam", H * d, torch.float32, required=False)
    _lib.need(db_lam, "db_lam", H, torch.float32, required=False)
    _lib.need_bytes(workspace, "workspace", 0)
    st = _lib.load().lion_backward(ctypes.byref(p), _ptr(x), _ptr(cu_seqlens), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                                   _ptr(w_lam), _ptr(b_lam), _ptr(act), _ptr(y), _ptr(dy), _ptr(dx), _ptr(dw_q),
                                   _ptr(dw_k), _ptr(dw_v), _ptr(dw_lam), _ptr(db_lam), _ptr(workspace),
                                   _nbytes(workspace), _stream(stream))
    _lib.check(st, "lion_backward")


def _check_inputs(x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam, num_heads, decay):
    torch = _torch()
    T, d = x.shape
    D = w_q.shape[1]
    if D % num_heads:
        raise ValueError("w_q columns must be a multiple of num_heads")
    checks = [("w_q", w_q, (d, D)), ("w_k", w_k, (d, D)), ("w_v", w_v, (d, D))]
    if decay == "s":
        checks.append(("w_lam", w_lam, (num_heads, d)))
    for name, t, shape in checks:
        if t is None or tuple(t.shape) != shape or t.dtype != x.dtype:
            raise ValueError(f"{name}: expected {shape} {x.dtype}")
    if decay in ("s", "d") and (b_lam is None or b_lam.dtype != torch.float32 or tuple(b_lam.shape) != (num_heads,)):
        raise ValueError("b_lam must be float32 [num_heads]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be int32 [N+1]")
    return problem(cu_seqlens.numel() - 1, T, d, num_heads, D // num_heads, x.dtype, decay)


def forward(x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam, num_heads: int, workspace=None,
            save_activations: bool = True, decay: str = "s"):
    """Allocate y, the activation cache (if save_activations) and the workspace
    (unless given) and run lion_forward. w_lam is used by decay "s" only, b_lam
    by "s" and "d" (pass None otherwise). Returns (y [T, H*d_h], act or None)."""
    torch = _torch()
    p = _check_inputs(x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam, num_heads, decay)
    dev = x.device
    y = torch.empty((p.total_tokens, p.num_heads * p.head_dim), dtype=x.dtype, device=dev)
    act = torch.empty(activation_size(p), dtype=torch.uint8, device=dev) if save_activations else None
    if workspace is None:
        workspace = torch.empty(workspace_size(p, False), dtype=torch.uint8, device=dev)
    lion_forward(p, x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam, y, act, workspace)
    return y, act


def backward(x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam, act, y, dy, num_heads: int, workspace=None,
             decay: str = "s") -> dict:
    """Allocate the gradients (and the workspace unless given) and run
    lion_backward. Returns dict dx, dw_q, dw_k, dw_v and, as the decay has
    them, dw_lam ("s") and db_lam ("s", "d")."""
    torch = _torch()
    p = _check_inputs(x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam, num_heads, decay)
    TD = (p.total_tokens, p.num_heads * p.head_dim)
    for name, t in (("y", y), ("dy", dy)):
        if tuple(t.shape) != TD or t.dtype != x.dtype:
            raise ValueError(f"{name}: expected {TD} {x.dtype}, got {tuple(t.shape)} {t.dtype}")
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty_like(x), dw_q=torch.empty(w_q.shape, **f32), dw_k=torch.empty(w_k.shape, **f32),
             dw_v=torch.empty(w_v.shape, **f32),
             dw_lam=torch.empty((num_heads, x.shape[1]), **f32) if decay == "s" else None,
             db_lam=torch.empty((num_heads,), **f32) if decay in ("s", "d") else None)
    if workspace is None:
        workspace = torch.empty(workspace_size(p, True), dtype=torch.uint8, device=dev)
    lion_backward(p, x, cu_seqlens, w_q, w_k, w_v, w_lam, b_lam, act, y, dy, g["dx"], g["dw_q"], g["dw_k"],
                  g["dw_v"], g["dw_lam"], g["db_lam"], workspace)
    return {k: v for k, v in g.items() if v is not None}
