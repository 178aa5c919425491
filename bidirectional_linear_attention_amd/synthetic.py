"""Seeded synthetic workloads for the GBLA and LION-s layers.

This module only draws random numbers and rounds them to the storage dtype.
It contains none of the layer's arithmetic, so the HIP path and the float64
oracle can both be fed from it without sharing any computation.

Shapes follow the long user-history encoders of "Gated Bidirectional Linear
Attention for Generative Retrieval" (Experimental setup, industrial setting:
head dim 64, Conv1D kernel 4; Table 5/6 benchmark: batch 8, L up to 32768) and
the LION-s selective-decay model of "Linear Attention for Efficient
Bidirectional Sequence Modeling" (three instantiations table, Lion-s).

Draw order (fixed, so a workload is a pure function of its seed):
  1. sequence lengths (ragged workloads only),
  2. x ~ N(0, 1)               [T, d]
  3. duplicated rows (repeated-interaction workloads only),
  4. conv_w ~ U(-0.5, 0.5)     [d, 4]
  5. W_Q, W_K, W_V ~ N(0, 1/d) [d, H*d_h]
  6. w_g ~ N(0, 1/d)           [H, d]   (w_lam for LION-s)
  7. dY ~ N(0, 1)              [T, H*d_h]
Values are then rounded to the storage dtype (round-to-nearest-even for bf16)
and kept as float32 arrays holding exactly representable values.

The gated RMSNorm output of the GBLA page's Eq. (7) draws its weights from a
second stream (seed + 7919), so turning it on leaves the draws above intact:
  W_R ~ N(0, 1/d) [d, H*d_h] (storage dtype), gamma ~ 1 + 0.1 N(0, 1) [d_h] (float32).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_output_gate", "round_bf16", "small_variant"]


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    try:  # torch's float32 -> bfloat16 cast is round-to-nearest-even and multi-threaded
        import torch
        return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    bits = a.view(np.uint32)
    # finite values never overflow 32 bits here: |bits| <= 0xFF7FFFFF, + 0x8000
    rounded = bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    rounded &= np.uint32(0xFFFF0000)
    return rounded.view(np.float32).reshape(a.shape)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    variant: str            # "gbla" or "lion"
    dtype: str              # "f32" or "bf16"
    d_model: int
    num_heads: int
    head_dim: int
    lengths: Optional[tuple] = None   # fixed lengths; None -> lognormal draw
    num_seqs: int = 0                 # for lognormal draws
    ln_median: float = 600.0
    ln_sigma: float = 1.0
    len_clip: tuple = (16, 32768)
    dup_frac: float = 0.0
    gate_bias: float = 0.0
    backward: bool = True
    chunk: int = 64                   # LION-s chunk length
    seed: int = 0

    @property
    def D(self) -> int:
        return self.num_heads * self.head_dim


WORKLOADS = {
    # single fp32 sequence, forward only
    "gbla_f32_L256_d64": Workload("gbla_f32_L256_d64", "gbla", "f32", 64, 1, 32,
                                  lengths=(256,), backward=False, seed=0),
    # 32 sequences of 1024 tokens, d=256, 4 heads
    "gbla_bf16_B32_L1024_d256": Workload("gbla_bf16_B32_L1024_d256", "gbla", "bf16", 256, 4, 64,
                                         lengths=(1024,) * 32, seed=1),
    # long-history encoder: 8 x 8192 tokens, d=512, 8 heads, 10% repeated rows, gate bias +1
    "gbla_bf16_B8_L8192_d512": Workload("gbla_bf16_B8_L8192_d512", "gbla", "bf16", 512, 8, 64,
                                        lengths=(8192,) * 8, dup_frac=0.1, gate_bias=1.0, seed=2),
    # the same recipe at the longest length of the latency benchmark: 8 x 32768 tokens
    "gbla_bf16_B8_L32768_d512": Workload("gbla_bf16_B8_L32768_d512", "gbla", "bf16", 512, 8, 64,
                                         lengths=(32768,) * 8, dup_frac=0.1, gate_bias=1.0, seed=5),
    # ragged packed batch: 256 lognormal lengths (median 600, sigma 1), clipped to [16, 32768]
    "gbla_bf16_ragged_N256_d512": Workload("gbla_bf16_ragged_N256_d512", "gbla", "bf16", 512, 8, 64,
                                           lengths=None, num_seqs=256, seed=3),
    # LION-s selective decay, 16 x 4096 tokens, chunk 64
    "lion_s_bf16_B16_L4096_d512": Workload("lion_s_bf16_B16_L4096_d512", "lion", "bf16", 512, 8, 64,
                                           lengths=(4096,) * 16, gate_bias=3.0, chunk=64, seed=4),
}


def small_variant(w: Workload, lengths, d_model=None, num_heads=None, head_dim=None,
                  dtype=None, seed=None) -> Workload:
    """Same recipe as `w` at a smaller shape (for parity tests the oracle finishes in seconds)."""
    return dataclasses.replace(
        w, name=w.name + "_small", lengths=tuple(int(n) for n in lengths),
        d_model=d_model or w.d_model, num_heads=num_heads or w.num_heads,
        head_dim=head_dim or w.head_dim, dtype=dtype or w.dtype,
        seed=w.seed if seed is None else seed)


def _lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.lengths is not None:
        return np.asarray(w.lengths, dtype=np.int64)
    raw = np.exp(rng.normal(np.log(w.ln_median), w.ln_sigma, size=w.num_seqs))
    return np.clip(np.rint(raw), w.len_clip[0], w.len_clip[1]).astype(np.int64)


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw one batch of the workload.

    Returns a dict of numpy arrays: x, cu_seqlens (int32), conv_w, w_q, w_k, w_v,
    w_g (or w_lam), b_g (or b_lam), dy, plus the integer sizes. Float arrays are
    float32 holding values exactly representable in the workload's dtype.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    lens = _lengths(w, rng)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    T, d, H, dh = int(cu[-1]), w.d_model, w.num_heads, w.head_dim
    D = H * dh

    x = rng.standard_normal((T, d), dtype=np.float32)
    if w.dup_frac > 0:
        for b in range(len(lens)):
            s, L = int(cu[b]), int(lens[b])
            n_dup = int(np.floor(w.dup_frac * L))
            if n_dup == 0 or L < 2:
                continue
            pos = np.sort(rng.choice(np.arange(1, L), size=min(n_dup, L - 1), replace=False))
            for t in pos:
                u = int(rng.integers(0, t))
                x[s + t] = x[s + u]
    conv_w = rng.uniform(-0.5, 0.5, size=(d, 4)).astype(np.float32)
    std = 1.0 / np.sqrt(d)
    w_q = (rng.standard_normal((d, D)) * std).astype(np.float32)
    w_k = (rng.standard_normal((d, D)) * std).astype(np.float32)
    w_v = (rng.standard_normal((d, D)) * std).astype(np.float32)
    w_g = (rng.standard_normal((H, d)) * std).astype(np.float32)
    b_g = np.full((H,), w.gate_bias, dtype=np.float32)
    dy = rng.standard_normal((T, D), dtype=np.float32)

    if w.dtype == "bf16":
        x, conv_w, w_q, w_k, w_v, w_g, dy = (round_bf16(a) for a in (x, conv_w, w_q, w_k, w_v, w_g, dy))
    out = dict(x=x, cu_seqlens=cu.astype(np.int32), conv_w=conv_w, w_q=w_q, w_k=w_k, w_v=w_v,
               dy=dy, T=T, N=len(lens), d=d, H=H, dh=dh, dtype=w.dtype)
    if w.variant == "lion":
        out["w_lam"], out["b_lam"] = w_g, b_g
    else:
        out["w_g"], out["b_g"] = w_g, b_g
    return out


def make_output_gate(w: Workload, seed: Optional[int] = None) -> dict:
    """Weights of the gated RMSNorm output for workload w: w_r [d, H*d_h]
    (values exact in the workload's dtype) and gamma [d_h] (float32)."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 7919)
    d, D = w.d_model, w.num_heads * w.head_dim
    w_r = (rng.standard_normal((d, D)) / np.sqrt(d)).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(w.head_dim)).astype(np.float32)
    if w.dtype == "bf16":
        w_r = round_bf16(w_r)
    return dict(w_r=w_r, gamma=gamma)
