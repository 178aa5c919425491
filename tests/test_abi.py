"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function declared in include/*.h, and rejects bad arguments before it
enqueues anything."""
import ctypes
import glob
import os
import re

import pytest

import bidirectional_linear_attention_amd as gb
from bidirectional_linear_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M):
            if not m.group(0).lstrip().startswith(("typedef", "#")):
                names.add(m.group(1))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = _lib.load()
    declared = _declared_functions()
    assert "gbla_forward" in declared and "gbla_backward" in declared
    missing = [n for n in declared if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings_and_version():
    lib = _lib.load()
    for code in range(7):
        assert lib.gbla_status_string(code).decode().startswith(_lib.STATUS[code])
    assert lib.gbla_version() >= 1


def _prob(**kw):
    base = dict(num_seqs=2, total_tokens=100, d_model=64, num_heads=2, head_dim=64, dtype=gb.DTYPE_BF16,
                output_gate=0, norm_eps=1e-6)
    base.update(kw)
    return gb.GblaProblem(base["num_seqs"], base["total_tokens"], base["d_model"], base["num_heads"],
                          base["head_dim"], base["dtype"], 0, 4, base["output_gate"], base["norm_eps"])


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=48), 3), (dict(dtype=7), 3), (dict(d_model=60), 2), (dict(num_seqs=0), 2),
    (dict(total_tokens=-1), 2), (dict(num_heads=0), 2), (dict(total_tokens=1 << 30), 2),
    (dict(output_gate=2), 3), (dict(output_gate=1, norm_eps=-1.0), 2), (dict(output_gate=1, norm_eps=float("nan")), 2),
    (dict(output_gate=1, norm_eps=float("inf")), 2),
    (dict(total_tokens=1, d_model=1 << 22, num_heads=8), 2),  # packed dX weights past 2^31 elements
    (dict(total_tokens=1, d_model=1 << 21, num_heads=1, head_dim=32), 2),  # rows past 32-bit buffer offsets
])
def test_size_queries_reject_bad_problems(kw, status):
    lib = _lib.load()
    out = ctypes.c_size_t()
    assert lib.gbla_workspace_size(ctypes.byref(_prob(**kw)), 0, ctypes.byref(out)) == status
    assert lib.gbla_saved_size(ctypes.byref(_prob(**kw)), ctypes.byref(out)) == status


def test_unsupported_gate_and_conv_width():
    lib = _lib.load()
    out = ctypes.c_size_t()
    p = _prob()
    p.gate = 2
    assert lib.gbla_workspace_size(ctypes.byref(p), 0, ctypes.byref(out)) == 3
    p = _prob()
    p.conv_width = 3
    assert lib.gbla_workspace_size(ctypes.byref(p), 1, ctypes.byref(out)) == 3


def test_softmax_gate_saved_size_adds_the_logit_maxima():
    """The softmax gate's saved buffer holds the states and then one logit
    maximum per (sequence, head)."""
    lib = _lib.load()
    out = ctypes.c_size_t()
    p = _prob()
    p.gate = _lib.GATE_SOFTMAX
    assert lib.gbla_saved_size(ctypes.byref(p), ctypes.byref(out)) == 0
    assert out.value == 4 * 2 * 2 * (64 * 64 + 64 + 1)
    assert lib.gbla_workspace_size(ctypes.byref(p), 0, ctypes.byref(out)) == 0
    soft = out.value
    p.gate = _lib.GATE_SIGMOID
    assert lib.gbla_workspace_size(ctypes.byref(p), 0, ctypes.byref(out)) == 0
    assert soft >= out.value


def test_size_queries_are_consistent():
    lib = _lib.load()
    out = ctypes.c_size_t()
    p = _prob()
    assert lib.gbla_saved_size(ctypes.byref(p), ctypes.byref(out)) == 0
    assert out.value == 4 * 2 * 2 * (64 * 64 + 64)
    assert lib.gbla_workspace_size(ctypes.byref(p), 0, ctypes.byref(out)) == 0
    fwd = out.value
    assert lib.gbla_workspace_size(ctypes.byref(p), 1, ctypes.byref(out)) == 0
    assert out.value > fwd > 0
    assert lib.gbla_workspace_size(None, 0, ctypes.byref(out)) == 1
    assert lib.gbla_workspace_size(ctypes.byref(p), 0, None) == 1
    assert lib.gbla_activation_size(ctypes.byref(p), ctypes.byref(out)) == 0
    # x~, phi(q), phi(k), v in bf16 and the gates in float32
    assert out.value >= 100 * (64 + 3 * 128) * 2 + 100 * 2 * 4


def _fake(addr=0x10000):
    return ctypes.c_void_p(addr)


def test_forward_rejects_null_misaligned_and_small_workspace_without_launching():
    lib = _lib.load()
    p = _prob()
    out = ctypes.c_size_t()
    lib.gbla_workspace_size(ctypes.byref(p), 0, ctypes.byref(out))
    need = out.value
    # x, cu, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma, y, saved, act (w_r, gamma NULL: plain output)
    a = [_fake(0x10000 + 0x1000 * i) for i in range(13)]
    a[8] = a[9] = None
    # NULL weight
    args = list(a)
    args[4] = None
    assert lib.gbla_forward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 1
    # misaligned x
    args = list(a)
    args[0] = _fake(0x10008)
    assert lib.gbla_forward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 4
    # workspace one byte short
    assert lib.gbla_forward(ctypes.byref(p), *a, _fake(0x900000), need - 1, None) == 5
    # bad problem is reported first
    bad = _prob(head_dim=16)
    assert lib.gbla_forward(ctypes.byref(bad), *a, _fake(0x900000), need, None) == 3
    # the plain output takes no W_R and no gamma
    args = list(a)
    args[9] = _fake(0x80000)
    assert lib.gbla_forward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 1


def test_forward_gated_output_argument_rules():
    lib = _lib.load()
    p = _prob(output_gate=1)
    out = ctypes.c_size_t()
    lib.gbla_workspace_size(ctypes.byref(p), 0, ctypes.byref(out))
    need = out.value
    a = [_fake(0x10000 + 0x1000 * i) for i in range(13)]
    args = list(a)
    args[8] = None    # W_R is required
    assert lib.gbla_forward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 1
    args = list(a)
    args[8] = _fake(0x18008)   # misaligned W_R
    assert lib.gbla_forward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 4
    args = list(a)
    args[9] = _fake(0x19002)   # misaligned gamma
    assert lib.gbla_forward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 4
    assert lib.gbla_forward(ctypes.byref(p), *a, _fake(0x900000), need - 1, None) == 5


def test_backward_rejects_null_and_small_workspace_without_launching():
    lib = _lib.load()
    p = _prob()
    out = ctypes.c_size_t()
    lib.gbla_workspace_size(ctypes.byref(p), 1, ctypes.byref(out))
    need = out.value
    # x, cu, conv_w, w_q, w_k, w_v, w_g, b_g, w_r, gamma, saved, act, dy, dx, dconv_w,
    # dw_q, dw_k, dw_v, dw_g, db_g, dw_r, dgamma
    a = [_fake(0x10000 + 0x1000 * i) for i in range(22)]
    a[8] = a[9] = a[20] = a[21] = None
    args = list(a)
    args[19] = None   # db_g
    assert lib.gbla_backward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 1
    assert lib.gbla_backward(ctypes.byref(p), *a, _fake(0x900000), need - 256, None) == 5


def test_backward_gated_output_argument_rules():
    lib = _lib.load()
    p = _prob(output_gate=1)
    out = ctypes.c_size_t()
    lib.gbla_workspace_size(ctypes.byref(p), 1, ctypes.byref(out))
    need = out.value
    a = [_fake(0x10000 + 0x1000 * i) for i in range(22)]
    for idx in (8, 20):           # W_R and dW_R are required
        args = list(a)
        args[idx] = None
        assert lib.gbla_backward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 1
    args = list(a)
    args[21] = None               # gamma given without dgamma
    assert lib.gbla_backward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 1
    args[9] = None                # neither: no RMSNorm scale
    assert lib.gbla_backward(ctypes.byref(p), *args, _fake(0x900000), need - 256, None) == 5


def test_gated_output_sizes():
    """The gated output adds the R segment: activations grow by T*H*d_h
    elements, and so does the gradient matrix in the backward workspace."""
    lib = _lib.load()
    out = ctypes.c_size_t()
    sizes = {}
    for og in (0, 1):
        p = _prob(output_gate=og)
        lib.gbla_activation_size(ctypes.byref(p), ctypes.byref(out))
        act = out.value
        lib.gbla_workspace_size(ctypes.byref(p), 1, ctypes.byref(out))
        sizes[og] = (act, out.value)
    assert sizes[1][0] - sizes[0][0] >= 100 * 128 * 2
    assert sizes[1][1] - sizes[0][1] >= 2 * (100 * 128 * 2)


# ---------------------------------------------------------------- LION-s entry points
def _lprob(**kw):
    base = dict(num_seqs=2, total_tokens=100, d_model=64, num_heads=2, head_dim=64, dtype=gb.DTYPE_BF16,
                chunk=64, decay=0)
    base.update(kw)
    return _lib.LionProblem(*(base[k] for k in ("num_seqs", "total_tokens", "d_model", "num_heads", "head_dim",
                                                "dtype", "chunk", "decay")))


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=48), 3), (dict(dtype=7), 3), (dict(chunk=32), 3), (dict(decay=3), 3), (dict(decay=-1), 3),
    (dict(d_model=60), 2), (dict(num_seqs=0), 2), (dict(total_tokens=-1), 2), (dict(num_heads=0), 2),
    (dict(total_tokens=1 << 30), 2), (dict(total_tokens=1, d_model=1 << 22, num_heads=8), 2),
    (dict(total_tokens=1, d_model=1 << 21, num_heads=1, head_dim=32), 2),
])
def test_lion_size_queries_reject_bad_problems(kw, status):
    lib = _lib.load()
    out = ctypes.c_size_t()
    assert lib.lion_workspace_size(ctypes.byref(_lprob(**kw)), 0, ctypes.byref(out)) == status
    assert lib.lion_activation_size(ctypes.byref(_lprob(**kw)), ctypes.byref(out)) == status


def test_lion_size_queries_are_consistent():
    lib = _lib.load()
    out = ctypes.c_size_t()
    p = _lprob()
    assert lib.lion_activation_size(ctypes.byref(p), ctypes.byref(out)) == 0
    act = out.value
    # raw q, k, v (bf16), log lambda and row sums, and two carried states per chunk slot and head
    slots = (100 + 63) // 64 + 2
    assert act >= 3 * 100 * 128 * 2 + 2 * 100 * 2 * 4 + slots * 2 * 2 * (64 * 64 + 64) * 4
    assert lib.lion_workspace_size(ctypes.byref(p), 0, ctypes.byref(out)) == 0
    assert out.value >= act
    assert lib.lion_workspace_size(ctypes.byref(p), 1, ctypes.byref(out)) == 0
    assert out.value > 0
    assert lib.lion_workspace_size(None, 0, ctypes.byref(out)) == 1
    assert lib.lion_activation_size(ctypes.byref(p), None) == 1


def test_lion_forward_rejects_bad_arguments_without_launching():
    lib = _lib.load()
    p = _lprob()
    out = ctypes.c_size_t()
    lib.lion_workspace_size(ctypes.byref(p), 0, ctypes.byref(out))
    need = out.value
    a = [_fake(0x10000 + 0x1000 * i) for i in range(9)]
    args = list(a)
    args[5] = None  # w_lam
    assert lib.lion_forward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 1
    args = list(a)
    args[2] = _fake(0x12004)  # misaligned w_q
    assert lib.lion_forward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 4
    assert lib.lion_forward(ctypes.byref(p), *a, _fake(0x900000), need - 1, None) == 5
    assert lib.lion_forward(ctypes.byref(_lprob(chunk=128)), *a, _fake(0x900000), need, None) == 3


def test_lion_backward_requires_the_activation_cache():
    lib = _lib.load()
    p = _lprob()
    out = ctypes.c_size_t()
    lib.lion_workspace_size(ctypes.byref(p), 1, ctypes.byref(out))
    need = out.value
    a = [_fake(0x10000 + 0x1000 * i) for i in range(16)]
    args = list(a)
    args[7] = None  # act
    assert lib.lion_backward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 1
    args = list(a)
    args[15] = _fake(0x1f002)  # misaligned db_lam
    assert lib.lion_backward(ctypes.byref(p), *args, _fake(0x900000), need, None) == 4
    assert lib.lion_backward(ctypes.byref(p), *a, _fake(0x900000), need - 256, None) == 5


@pytest.mark.parametrize("decay,null_ok,null_bad", [
    (1, [5], [6]),        # Lion-d: no w_lam; b_lam (the per-head logit) required
    (2, [5, 6], []),      # Lion-lit: neither
])
def test_lion_fixed_and_no_decay_argument_rules(decay, null_ok, null_bad):
    """w_lam (argument 5) and b_lam (6) may be NULL where the decay does not use
    them; the forward then only fails on the workspace size (nothing launched)."""
    lib = _lib.load()
    p = _lprob(decay=decay)
    out = ctypes.c_size_t()
    assert lib.lion_workspace_size(ctypes.byref(p), 0, ctypes.byref(out)) == 0
    need = out.value
    a = [_fake(0x10000 + 0x1000 * i) for i in range(9)]
    args = list(a)
    for i in null_ok:
        args[i] = None
    assert lib.lion_forward(ctypes.byref(p), *args, _fake(0x900000), need - 1, None) == 5
    for i in null_bad:
        bad = list(a)
        bad[i] = None
        assert lib.lion_forward(ctypes.byref(p), *bad, _fake(0x900000), need, None) == 1


class _FakeDev:
    """Stands in for a device tensor in the binding's host-side checks (no GPU here)."""

    def __init__(self, n, dtype, cuda=True, contiguous=True, esz=None):
        import torch
        self._n, self.dtype, self.is_cuda, self._c = n, dtype, cuda, contiguous
        self._esz = esz if esz is not None else torch.empty(0, dtype=dtype).element_size()

    def numel(self):
        return self._n

    def element_size(self):
        return self._esz

    def is_contiguous(self):
        return self._c


def test_binding_checks_dtype_device_and_size_before_launch():
    """The Python binding refuses, before any launch, a tensor of the wrong dtype,
    off the GPU, non-contiguous or smaller than the problem needs (a kernel would
    otherwise read or write past its end)."""
    import torch
    _lib.need(_FakeDev(10, torch.bfloat16), "dy", 10, torch.bfloat16)
    _lib.need(None, "w_r", 10, torch.bfloat16, required=False)
    bad = [(_FakeDev(9, torch.bfloat16), torch.bfloat16), (_FakeDev(10, torch.float32), torch.bfloat16),
           (_FakeDev(10, torch.bfloat16, cuda=False), torch.bfloat16),
           (_FakeDev(10, torch.bfloat16, contiguous=False), torch.bfloat16), (None, torch.bfloat16)]
    for t, dt in bad:
        with pytest.raises(ValueError):
            _lib.need(t, "dy", 10, dt)
    _lib.need_bytes(_FakeDev(100, torch.uint8), "act", 100)
    with pytest.raises(ValueError):
        _lib.need_bytes(_FakeDev(99, torch.uint8), "act", 100)
    with pytest.raises(ValueError):
        _lib.need_bytes(None, "act", 1)
    assert _lib._torch_dtype(_lib.DTYPE_BF16) == torch.bfloat16 and _lib._torch_dtype(_lib.DTYPE_F32) == torch.float32


def test_gbla_binding_rejects_mismatched_gradient_buffers():
    """gbla_backward's binding checks dy, saved and the activation cache against
    the problem: a bf16/float32 mix-up, a narrower dy or a short cache raises
    ValueError before the library is called."""
    import torch
    import bidirectional_linear_attention_amd as gb
    p = gb.problem(2, 64, 32, 2, 32, torch.bfloat16)
    T, d, D = 64, 32, 64
    bf, f32 = torch.bfloat16, torch.float32
    ok = dict(x=_FakeDev(T * d, bf), cu_seqlens=_FakeDev(3, torch.int32), conv_w=_FakeDev(d * 4, bf),
              w_q=_FakeDev(d * D, bf), w_k=_FakeDev(d * D, bf), w_v=_FakeDev(d * D, bf), w_g=_FakeDev(2 * d, bf),
              b_g=_FakeDev(2, f32), saved=_FakeDev(gb.saved_size(p) // 4, f32),
              act=_FakeDev(gb.activation_size(p), torch.uint8), dy=_FakeDev(T * D, bf), dx=_FakeDev(T * d, bf),
              dconv_w=_FakeDev(d * 4, f32), dw_q=_FakeDev(d * D, f32), dw_k=_FakeDev(d * D, f32),
              dw_v=_FakeDev(d * D, f32), dw_g=_FakeDev(2 * d, f32), db_g=_FakeDev(2, f32))
    for key, t in (("dy", _FakeDev(T * D, f32)), ("dy", _FakeDev(T * D - 1, bf)), ("saved", _FakeDev(10**6, bf)),
                   ("act", _FakeDev(gb.activation_size(p) - 1, torch.uint8)), ("dx", _FakeDev(T * d, f32))):
        kw = dict(ok)
        kw[key] = t
        with pytest.raises(ValueError, match=key):
            gb.gbla_backward(p, kw["x"], kw["cu_seqlens"], kw["conv_w"], kw["w_q"], kw["w_k"], kw["w_v"],
                             kw["w_g"], kw["b_g"], kw["saved"], kw["act"], kw["dy"], kw["dx"], kw["dconv_w"],
                             kw["dw_q"], kw["dw_k"], kw["dw_v"], kw["dw_g"], kw["db_g"], workspace=None)


def test_noalloc_forward_refuses_problems_beyond_its_scratch_without_launching():
    """gbla_forward_noalloc checks its static scratch limit on the host, before
    touching the device: without an activation cache the activations count too."""
    lib = _lib.load()
    p = _prob(total_tokens=300_000)
    out = ctypes.c_size_t()
    assert lib.gbla_workspace_size(ctypes.byref(p), 0, ctypes.byref(out)) == 0
    assert out.value > _lib.STATIC_SCRATCH_BYTES
    args = [_fake(0x10000 + 0x1000 * i) for i in range(13)]
    args[8] = args[9] = None  # w_r, gamma (plain output)
    args[12] = None  # act
    assert lib.gbla_forward_noalloc(ctypes.byref(p), *args, None) == 7
    assert lib.gbla_status_string(7).decode().startswith("GBLA_ERR_SCRATCH_LIMIT")
