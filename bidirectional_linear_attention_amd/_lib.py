"""ctypes view of libgbla.so (include/gbla.h, include/lion.h). Marshalling only: every step of
the layer runs in the HIP library; there is no CPU or PyTorch fallback."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# GBLA_LIBRARY may name another build of the same library (e.g. to compare two builds)
LIB_PATH = os.environ.get("GBLA_LIBRARY") or os.path.join(_PKG, "libgbla.so")

STATUS = {
    0: "GBLA_OK", 1: "GBLA_ERR_NULL_ARG", 2: "GBLA_ERR_BAD_SHAPE", 3: "GBLA_ERR_UNSUPPORTED",
    4: "GBLA_ERR_MISALIGNED", 5: "GBLA_ERR_WORKSPACE_TOO_SMALL", 6: "GBLA_ERR_HIP", 7: "GBLA_ERR_SCRATCH_LIMIT",
}
# bytes of the static scratch array of gbla_forward_noalloc (GBLA_STATIC_SCRATCH_BYTES in include/gbla.h)
STATIC_SCRATCH_BYTES = 128 << 20
DTYPE_F32, DTYPE_BF16 = 0, 1
LION_DECAY = {"s": 0, "d": 1, "lit": 2}  # selective, fixed per head, none
GATE_SIGMOID = 0
GATE_SOFTMAX = 1
GATES = {"sigmoid": GATE_SIGMOID, "softmax": GATE_SOFTMAX}
OUTPUT_PLAIN, OUTPUT_GATED_RMSNORM = 0, 1


class GblaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class GblaProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("num_seqs", "total_tokens", "d_model", "num_heads", "head_dim", "dtype", "gate", "conv_width",
                 "output_gate")] + [("norm_eps", ctypes.c_float)]


class LionProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("num_seqs", "total_tokens", "d_model", "num_heads", "head_dim", "dtype", "chunk", "decay")]


_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_P = ctypes.POINTER(GblaProblem)
_LP = ctypes.POINTER(LionProblem)

_SIGNATURES = {
    "gbla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gbla_version": (ctypes.c_int, []),
    "gbla_saved_size": (ctypes.c_int, [_P, ctypes.POINTER(_sz)]),
    "gbla_workspace_size": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(_sz)]),
    "gbla_activation_size": (ctypes.c_int, [_P, ctypes.POINTER(_sz)]),
    "gbla_forward": (ctypes.c_int, [_P] + [_vp] * 13 + [_vp, _sz, _vp]),
    "gbla_forward_noalloc": (ctypes.c_int, [_P] + [_vp] * 13 + [_vp]),
    "gbla_backward": (ctypes.c_int, [_P] + [_vp] * 22 + [_vp, _sz, _vp]),
    "gbla_profile_begin": (ctypes.c_int, [ctypes.c_int]),
    "gbla_profile_begin_stages": (ctypes.c_int, [ctypes.c_int, ctypes.c_uint64]),
    "gbla_profile_end": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int),
                                        ctypes.c_int, ctypes.POINTER(ctypes.c_int)]),
    "gbla_profile_stage_name": (ctypes.c_char_p, [ctypes.c_int]),
    "lion_workspace_size": (ctypes.c_int, [_LP, ctypes.c_int, ctypes.POINTER(_sz)]),
    "lion_activation_size": (ctypes.c_int, [_LP, ctypes.POINTER(_sz)]),
    "lion_forward": (ctypes.c_int, [_LP] + [_vp] * 9 + [_vp, _sz, _vp]),
    "lion_backward": (ctypes.c_int, [_LP] + [_vp] * 16 + [_vp, _sz, _vp]),
}

_lib = None


def load():
    """Load libgbla.so once. torch is imported first so the library binds to the
    same HIP runtime instance as torch's device memory and streams."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m bidirectional_linear_attention_amd.build` (no fallback path exists)")
    import torch  # noqa: F401  (shares the HIP runtime)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        if not hasattr(lib, name):
            continue
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def check(status: int, where: str):
    if status != 0:
        raise GblaError(status, where)


def _torch_dtype(code: int):
    import torch
    return torch.bfloat16 if code == DTYPE_BF16 else torch.float32


def need(t, name: str, nelem: int, dtype, required: bool = True) -> None:
    """Host-side guard before a launch: tensor t (None allowed unless required)
    must have the given torch dtype, live on the GPU, be contiguous and hold at
    least nelem elements, so that no kernel reads or writes past its end."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous GPU tensor")
    if t.numel() < nelem:
        raise ValueError(f"{name}: needs at least {nelem} elements, got {t.numel()}")


def need_bytes(t, name: str, nbytes: int, required: bool = True) -> None:
    """As need(), for byte buffers (activation cache, workspace) of any dtype."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous GPU tensor")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: needs at least {nbytes} bytes, got {t.numel() * t.element_size()}")

