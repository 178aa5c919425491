"""MI355X-native Gated Bidirectional Linear Attention (GBLA).

Python binding of libgbla.so (C ABI in include/gbla.h). The functions named
like the C entry points take torch tensors and pass their device pointers and
the current HIP stream; the convenience wrappers `forward` / `backward` also
allocate the outputs and the workspace. Every step of the layer runs in the
library's HIP kernels; if the library is missing an error is raised.

The layer is Eqs. (4)-(6) of "Gated Bidirectional Linear Attention for
Generative Retrieval" (core method): causal depthwise Conv1d (kernel 4), per-head
Q/K/V projections, phi = elu + 1, key gate (per-token sigmoid, or the softmax
over the sequence that Eq. (5) writes), global state
S = sum_j g_j phi(k_j) v_j^T, z = sum_j g_j phi(k_j), readout
O_i = phi(q_i)^T S / phi(q_i)^T z, optionally followed by the gated RMSNorm
output of Eq. (7), y = gamma * RmsNorm(O) * SiLU(x~ W_R), on packed
variable-length sequences.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import DTYPE_BF16, DTYPE_F32, GATES, OUTPUT_GATED_RMSNORM, OUTPUT_PLAIN, GblaError, GblaProblem

__all__ = ["GblaProblem", "GblaError", "problem", "saved_size", "workspace_size", "activation_size", "gbla_forward",
           "gbla_forward_noalloc", "gbla_backward", "forward", "backward", "profile_begin", "profile_end", "stage_names", "DTYPE_F32", "DTYPE_BF16"]


def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return DTYPE_F32
    if dt == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {dt}: float32 or bfloat16")


def problem(num_seqs: int, total_tokens: int, d_model: int, num_heads: int, head_dim: int, dtype,
            gate: str = "sigmoid", gated_output: bool = False, norm_eps: float = 1e-6) -> GblaProblem:
    """Problem descriptor; dtype is a torch dtype or a DTYPE_* code, gate
    "sigmoid" or "softmax"; gated_output selects the gated RMSNorm output of
    Eq. (7) with RMSNorm epsilon norm_eps."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return GblaProblem(int(num_seqs), int(total_tokens), int(d_model), int(num_heads), int(head_dim), code,
                       GATES[gate], 4, OUTPUT_GATED_RMSNORM if gated_output else OUTPUT_PLAIN, float(norm_eps))


def saved_size(p: GblaProblem) -> int:
    out = ctypes.c_size_t()
    _lib.check(_lib.load().gbla_saved_size(ctypes.byref(p), ctypes.byref(out)), "gbla_saved_size")
    return out.value


def workspace_size(p: GblaProblem, backward: bool) -> int:
    out = ctypes.c_size_t()
    _lib.check(_lib.load().gbla_workspace_size(ctypes.byref(p), int(bool(backward)), ctypes.byref(out)),
               "gbla_workspace_size")
    return out.value


def activation_size(p: GblaProblem) -> int:
    out = ctypes.c_size_t()
    _lib.check(_lib.load().gbla_activation_size(ctypes.byref(p), ctypes.byref(out)), "gbla_activation_size")
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


def _check_common(p: GblaProblem, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma) -> None:
    """Sizes and dtypes of the arguments the forward and backward share, against p."""
    torch = _torch()
    dt = _lib._torch_dtype(p.dtype)
    T, d, H, D = p.total_tokens, p.d_model, p.num_heads, p.num_heads * p.head_dim
    _lib.need(x, "x", T * d, dt, required=T > 0)
    _lib.need(cu_seqlens, "cu_seqlens", p.num_seqs + 1, torch.int32)
    _lib.need(conv_w, "conv_w", d * 4, dt)
    for name, w in (("w_q", w_q), ("w_k", w_k), ("w_v", w_v)):
        _lib.need(w, name, d * D, dt)
    _lib.need(w_g, "w_g", H * d, dt)
    _lib.need(b_g, "b_g", H, torch.float32)
    _lib.need(w_r, "w_r", d * D, dt, required=False)
    _lib.need(gamma, "gamma", p.head_dim, torch.float32, required=False)


def gbla_forward(p: GblaProblem, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, y, saved, act, workspace,
                 stream=None, w_r=None, gamma=None) -> None:
    """Enqueue the forward pass (include/gbla.h: gbla_forward); act may be None;
    w_r (and optionally gamma) for the gated RMSNorm output. Every tensor is
    checked against p (dtype, device, size) before anything is enqueued."""
    torch = _torch()
    _check_common(p, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma)
    _lib.need(y, "y", p.total_tokens * p.num_heads * p.head_dim, _lib._torch_dtype(p.dtype),
              required=p.total_tokens > 0)
    _lib.need(saved, "saved", saved_size(p) // 4, torch.float32)
    _lib.need_bytes(act, "act", activation_size(p), required=False)
    _lib.need_bytes(workspace, "workspace", 0)
    st = _lib.load().gbla_forward(ctypes.byref(p), _ptr(x), _ptr(cu_seqlens), _ptr(conv_w), _ptr(w_q), _ptr(w_k),
                                  _ptr(w_v), _ptr(w_g), _ptr(b_g), _ptr(w_r), _ptr(gamma), _ptr(y), _ptr(saved),
                                  _ptr(act), _ptr(workspace),
                                  ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(stream))
    _lib.check(st, "gbla_forward")


def gbla_forward_noalloc(p: GblaProblem, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, y, saved, act,
                         stream=None, w_r=None, gamma=None) -> None:
    """Enqueue the allocation-free forward (include/gbla.h: gbla_forward_noalloc):
    gbla_forward without a workspace argument, its scratch being the library's
    static device array. Calls on one GPU share that array, so calls that
    overlap in time on one GPU race. Same checks as gbla_forward."""
    torch = _torch()
    _check_common(p, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma)
    _lib.need(y, "y", p.total_tokens * p.num_heads * p.head_dim, _lib._torch_dtype(p.dtype),
              required=p.total_tokens > 0)
    _lib.need(saved, "saved", saved_size(p) // 4, torch.float32)
    _lib.need_bytes(act, "act", activation_size(p), required=False)
    st = _lib.load().gbla_forward_noalloc(ctypes.byref(p), _ptr(x), _ptr(cu_seqlens), _ptr(conv_w), _ptr(w_q),
                                          _ptr(w_k), _ptr(w_v), _ptr(w_g), _ptr(b_g), _ptr(w_r), _ptr(gamma),
                                          _ptr(y), _ptr(saved), _ptr(act), _stream(stream))
    _lib.check(st, "gbla_forward_noalloc")


def gbla_backward(p: GblaProblem, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, saved, act, dy, dx, dconv_w,
                  dw_q, dw_k, dw_v, dw_g, db_g, workspace, stream=None, w_r=None, gamma=None, dw_r=None,
                  dgamma=None) -> None:
    """Enqueue the backward pass (include/gbla.h: gbla_backward); act None
    recomputes. Every tensor is checked against p (dtype, device, size) before
    anything is enqueued."""
    torch = _torch()
    dt = _lib._torch_dtype(p.dtype)
    T, d, H, D = p.total_tokens, p.d_model, p.num_heads, p.num_heads * p.head_dim
    _check_common(p, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma)
    _lib.need(saved, "saved", saved_size(p) // 4, torch.float32)
    _lib.need_bytes(act, "act", activation_size(p), required=False)
    _lib.need(dy, "dy", T * D, dt, required=T > 0)
    _lib.need(dx, "dx", T * d, dt, required=T > 0)
    _lib.need(dconv_w, "dconv_w", d * 4, torch.float32)
    for name, t in (("dw_q", dw_q), ("dw_k", dw_k), ("dw_v", dw_v)):
        _lib.need(t, name, d * D, torch.float32)
    _lib.need(dw_g, "dw_g", H * d, torch.float32)
    _lib.need(db_g, "db_g", H, torch.float32)
    _lib.need(dw_r, "dw_r", d * D, torch.float32, required=False)
    _lib.need(dgamma, "dgamma", p.head_dim, torch.float32, required=False)
    _lib.need_bytes(workspace, "workspace", 0)
    st = _lib.load().gbla_backward(ctypes.byref(p), _ptr(x), _ptr(cu_seqlens), _ptr(conv_w), _ptr(w_q), _ptr(w_k),
                                   _ptr(w_v), _ptr(w_g), _ptr(b_g), _ptr(w_r), _ptr(gamma), _ptr(saved), _ptr(act),
                                   _ptr(dy), _ptr(dx), _ptr(dconv_w), _ptr(dw_q), _ptr(dw_k), _ptr(dw_v),
                                   _ptr(dw_g), _ptr(db_g), _ptr(dw_r), _ptr(dgamma), _ptr(workspace),
                                   ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(stream))
    _lib.check(st, "gbla_backward")


def _check_inputs(x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, num_heads, gate, w_r=None, gamma=None,
                  norm_eps=1e-6):
    torch = _torch()
    T, d = x.shape
    D = w_q.shape[1]
    if D % num_heads:
        raise ValueError("w_q columns must be a multiple of num_heads")
    mats = [("conv_w", conv_w, (d, 4)), ("w_q", w_q, (d, D)), ("w_k", w_k, (d, D)), ("w_v", w_v, (d, D)),
            ("w_g", w_g, (num_heads, d))]
    if w_r is not None:
        mats.append(("w_r", w_r, (d, D)))
    for name, t, shape in mats:
        if tuple(t.shape) != shape or t.dtype != x.dtype:
            raise ValueError(f"{name}: expected {shape} {x.dtype}, got {tuple(t.shape)} {t.dtype}")
    if b_g.dtype != torch.float32 or tuple(b_g.shape) != (num_heads,):
        raise ValueError("b_g must be float32 [num_heads]")
    if gamma is not None and (w_r is None or gamma.dtype != torch.float32 or tuple(gamma.shape) != (D // num_heads,)):
        raise ValueError("gamma must be float32 [head_dim] and needs w_r")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be int32 [N+1]")
    return problem(cu_seqlens.numel() - 1, T, d, num_heads, D // num_heads, x.dtype, gate, w_r is not None, norm_eps)


def forward(x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, num_heads: int, workspace=None,
            save_activations: bool = True, gate: str = "sigmoid", w_r=None, gamma=None, norm_eps: float = 1e-6):
    """Allocate y, saved, the activation cache (if save_activations) and the
    workspace (unless given) and run gbla_forward; w_r [d, H*d_h] (and
    optionally gamma [d_h] float32) selects the gated RMSNorm output.
    Returns (y [T, H*d_h], saved, act or None); saved is float32
    [N, H, d_h*d_h + d_h] for the sigmoid gate and flat (states, then the N*H
    logit maxima, as gbla_saved_size describes) for the softmax gate."""
    torch = _torch()
    p = _check_inputs(x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, num_heads, gate, w_r, gamma, norm_eps)
    dev = x.device
    y = torch.empty((p.total_tokens, p.num_heads * p.head_dim), dtype=x.dtype, device=dev)
    E = p.head_dim * p.head_dim + p.head_dim
    shape = (p.num_seqs, p.num_heads, E) if gate == "sigmoid" else (p.num_seqs * p.num_heads * (E + 1),)
    saved = torch.empty(shape, dtype=torch.float32, device=dev)
    act = torch.empty(activation_size(p), dtype=torch.uint8, device=dev) if save_activations else None
    if workspace is None:
        workspace = torch.empty(workspace_size(p, False), dtype=torch.uint8, device=dev)
    gbla_forward(p, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, y, saved, act, workspace, w_r=w_r, gamma=gamma)
    return y, saved, act


def backward(x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, saved, act, dy, num_heads: int,
             workspace=None, gate: str = "sigmoid", w_r=None, gamma=None, norm_eps: float = 1e-6) -> dict:
    """Allocate the gradients (and the workspace unless given) and run
    gbla_backward; act is forward's activation cache or None (recompute).
    Returns dict dx, dconv_w, dw_q, dw_k, dw_v, dw_g, db_g, plus dw_r (and
    dgamma) with the gated RMSNorm output."""
    torch = _torch()
    p = _check_inputs(x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, num_heads, gate, w_r, gamma, norm_eps)
    if saved.dtype != torch.float32 or saved.numel() * 4 != saved_size(p):
        raise ValueError("saved does not match the problem (float32; gate?)")
    if tuple(dy.shape) != (p.total_tokens, p.num_heads * p.head_dim) or dy.dtype != x.dtype:
        raise ValueError(f"dy: expected {(p.total_tokens, p.num_heads * p.head_dim)} {x.dtype}, "
                         f"got {tuple(dy.shape)} {dy.dtype}")
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty_like(x), dconv_w=torch.empty(conv_w.shape, **f32), dw_q=torch.empty(w_q.shape, **f32),
             dw_k=torch.empty(w_k.shape, **f32), dw_v=torch.empty(w_v.shape, **f32),
             dw_g=torch.empty(w_g.shape, **f32), db_g=torch.empty(b_g.shape, **f32))
    if workspace is None:
        workspace = torch.empty(workspace_size(p, True), dtype=torch.uint8, device=dev)
    if w_r is not None:
        g["dw_r"] = torch.empty(w_r.shape, **f32)
    if gamma is not None:
        g["dgamma"] = torch.empty(gamma.shape, **f32)
    gbla_backward(p, x, cu_seqlens, conv_w, w_q, w_k, w_v, w_g, b_g, saved, act, dy, g["dx"], g["dconv_w"],
                  g["dw_q"], g["dw_k"], g["dw_v"], g["dw_g"], g["db_g"], workspace, w_r=w_r, gamma=gamma,
                  dw_r=g.get("dw_r"), dgamma=g.get("dgamma"))
    return g


def stage_names() -> list:
    """Names of the profiled stages, in stage-id order."""
    lib = _lib.load()
    names = []
    for i in range(64):
        n = lib.gbla_profile_stage_name(i).decode()
        if n == "unknown":
            break
        names.append(n)
    return names


def profile_begin(max_records: int, stages=None) -> None:
    """Open the library's per-stage event-timing window; stages: iterable of
    stage names to time (None: all), see stage_names()."""
    lib = _lib.load()
    if stages is None:
        _lib.check(lib.gbla_profile_begin(int(max_records)), "gbla_profile_begin")
        return
    ids = {n: i for i, n in enumerate(stage_names())}
    mask = 0
    for n in stages:
        mask |= 1 << ids[n]
    _lib.check(lib.gbla_profile_begin_stages(int(max_records), ctypes.c_uint64(mask)), "gbla_profile_begin_stages")


def profile_end() -> dict:
    """Close the timing window; returns {stage name: (total device ms, launches)}."""
    lib = _lib.load()
    ms = (ctypes.c_double * 64)()
    n = (ctypes.c_int * 64)()
    ns = ctypes.c_int()
    _lib.check(lib.gbla_profile_end(ms, n, 64, ctypes.byref(ns)), "gbla_profile_end")
    return {lib.gbla_profile_stage_name(i).decode(): (ms[i], n[i]) for i in range(ns.value) if n[i] > 0}
