"""GPU parity of the HIP LION-s path (chunkwise, 64-token chunks) against the
float64 oracle's full masked-matrix form.

Every case feeds the same seeded inputs (bf16-representable values for bf16
workloads) to libgbla.so through the C ABI (include/lion.h) and to oracle.lion,
and compares each output with the max-norm relative error
    ||gpu - oracle||_inf / ||oracle||_inf
against 1e-4 for float32 inputs and 2e-2 for bfloat16 inputs with float32
accumulation. At the full 16 x 4096 size the oracle evaluates sampled
sequences (y and dx of a sequence depend only on that sequence), and the
weight gradients are checked through an identity that holds at any size.
"""
import numpy as np
import pytest
import torch

from bidirectional_linear_attention_amd import lion as gl
from bidirectional_linear_attention_amd.synthetic import WORKLOADS, make_inputs, small_variant
from oracle import lion as ol

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
GRADS = ("dx", "dw_q", "dw_k", "dw_v", "dw_lam", "db_lam")
LION = WORKLOADS["lion_s_bf16_B16_L4096_d512"]


def rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / max(den, 1e-30))


def sum_err(got, ref, terms):
    """Error of a per-head sum over tokens (db_lam = sum_t da_t) relative to the
    size of the summed terms, max over heads of sum_t |da_t|. The terms cancel
    (strongly so when the decay is strong), so a rounding difference of one ulp
    in a term moves the sum by ~1e-7 of that size, which the max-norm relative
    error of the small result can amplify past any fixed bound."""
    scale = max(float(np.max(np.abs(terms).sum(axis=0))), float(np.max(np.abs(ref))), 1e-30)
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)))) / scale


def to_dev(inp):
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt).contiguous()

    return dict(x=t(inp["x"]), cu=torch.from_numpy(inp["cu_seqlens"]).to("cuda"), w_q=t(inp["w_q"]),
                w_k=t(inp["w_k"]), w_v=t(inp["w_v"]), w_lam=t(inp["w_lam"]),
                b_lam=torch.from_numpy(inp["b_lam"]).float().to("cuda"), dy=t(inp["dy"]))


def run_gpu(inp, backward=True):
    d = to_dev(inp)
    H = inp["H"]
    y, act = gl.forward(d["x"], d["cu"], d["w_q"], d["w_k"], d["w_v"], d["w_lam"], d["b_lam"], H,
                        save_activations=backward)
    out = {"y": y}
    if backward:
        out.update(gl.backward(d["x"], d["cu"], d["w_q"], d["w_k"], d["w_v"], d["w_lam"], d["b_lam"], act, y,
                               d["dy"], H))
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in out.items()}


def oracle_args(inp):
    return [inp[k] for k in ("x", "cu_seqlens", "w_q", "w_k", "w_v", "w_lam", "b_lam")]


def grad_errors(gpu, g, keys, db_sum=False):
    """Max-norm relative error of every gradient in keys. db_lam is reported
    both ways: its plain max-norm relative error ("db_lam") and, as
    "db_lam_sum", its error relative to the summed terms (sum_err). The bound
    applies to the plain error unless db_sum is set; db_sum is for a strong
    decay, where the terms of db_lam = sum_t da_t cancel so much that one ulp in
    a term moves the small sum past a fixed relative bound."""
    errs = {}
    for k in keys:
        errs[k] = rel_err(gpu[k], g[k])
        if k == "db_lam":
            errs["db_lam_sum"] = sum_err(gpu[k], g[k], g["da"])
            # how strongly the sum cancels: sum_t |da_t| over |sum_t da_t| (largest head)
            errs["db_lam_cancel"] = float(np.max(np.abs(g["da"]).sum(axis=0)) / max(np.max(np.abs(g[k])), 1e-30))
    bounded = {k: v for k, v in errs.items() if k not in ("db_lam_cancel", "db_lam" if db_sum else "db_lam_sum")}
    return errs, bounded


def compare(inp, backward=True, tol=None, label="", db_sum=False):
    tol = TOL[inp["dtype"]] if tol is None else tol
    gpu = run_gpu(inp, backward)
    errs = {"y": rel_err(gpu["y"], ol.forward_full(*oracle_args(inp), inp["H"]))}
    bounded = dict(errs)
    if backward:
        g = ol.backward_full(*oracle_args(inp), inp["dy"], inp["H"])
        e, b = grad_errors(gpu, g, GRADS, db_sum)
        errs.update(e)
        bounded.update(b)
    print(f"\n[{label}] T={inp['T']} N={inp['N']} d={inp['d']} H={inp['H']} dh={inp['dh']} {inp['dtype']}: "
          + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in bounded.items() if not v <= tol}
    assert not bad, f"tolerance {tol} exceeded: {bad}"
    return gpu


# ------------------------------------------------------------ float32 parity at 1e-4

@pytest.mark.parametrize("lengths,d,H,dh", [
    ((300, 1, 130, 64, 65), 96, 3, 64),     # several chunks, ragged tails, one-token and exact-chunk sequences
    ((129, 0, 255, 40, 2), 64, 2, 32),      # empty sequence, head_dim 32
    ((512,), 40, 1, 64),                    # d not a multiple of the GEMM k chunk
    ((200, 65), 576, 10, 32),               # d > 512, H > 8: second channel and head groups of the decay logits
])
def test_f32_forward_backward_multi_chunk(lengths, d, H, dh):
    w = small_variant(LION, lengths, d_model=d, num_heads=H, head_dim=dh, dtype="f32", seed=51)
    compare(make_inputs(w), label="f32 " + str(lengths))


@pytest.mark.parametrize("bias", [-3.0, 12.0])
def test_f32_strong_and_vanishing_decay(bias):
    """bias -3: lambda ~ 0.05, the mask decays to ~0 within a few tokens (every
    exponent stays <= 0, nothing overflows); bias 12: lambda ~ 1 - 6e-6, almost
    the all-ones mask of Lion-lit. With the strong decay, db_lam is a strongly
    cancelling sum and is held to the size of its terms (both errors printed)."""
    w = small_variant(LION, (400, 70), d_model=64, num_heads=2, dtype="f32", seed=52)
    inp = make_inputs(w)
    inp["b_lam"] = np.full_like(inp["b_lam"], bias)
    compare(inp, label=f"f32 bias {bias}", db_sum=bias < 0)


# ------------------------------------------------------------ sequences of many chunks, every gradient

# 17, 33, 71 and 1 chunks of 64 tokens: the forward scan walks a sequence's
# chunks in rounds of 16 and the backward suffix sum in rounds of 64, so these
# lengths take every carry across one, two and four scan rounds and across a
# suffix round, with ragged last chunks
LONG = (1025, 2100, 4500, 30)


@pytest.mark.timeout(300)  # the float64 oracle takes ~10 s per case
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_chunks_every_gradient(dtype):
    w = small_variant(LION, LONG, d_model=128, num_heads=2, dtype=dtype, seed=70)
    compare(make_inputs(w), label=f"{dtype} LION-s 17/33/71-chunk sequences")


# ------------------------------------------------------------ bf16, the workload recipe at L <= 512

def test_bf16_small_recipe_L512():
    w = small_variant(LION, (512, 512, 200, 77), seed=53)
    compare(make_inputs(w), label="bf16 LION-s recipe L<=512")


def test_bf16_odd_head_count():
    w = small_variant(LION, (300, 77, 130), d_model=96, num_heads=3, seed=58)
    compare(make_inputs(w), label="bf16 LION-s H=3")


def test_bf16_small_ragged():
    w = small_variant(LION, (1, 63, 64, 65, 127, 128, 129, 450), d_model=128, num_heads=2, seed=54)
    compare(make_inputs(w), label="bf16 ragged chunks")


def test_bf16_head_dim_32():
    """head_dim 32 in bf16: one state quad per lane in the staging of the carried
    states, two 16-wide column tiles per output, several chunks and ragged tails."""
    w = small_variant(LION, (200, 64, 1, 130), d_model=96, num_heads=3, head_dim=32, seed=61)
    compare(make_inputs(w), label="bf16 LION-s dh=32")


# ------------------------------------------------------------ full size: 16 x 4096, d 512, 8 heads

@pytest.mark.timeout(400)  # the float64 oracle needs about a minute for one 4096-token sequence
def test_bf16_full_size_sampled_sequence_and_identity():
    inp = make_inputs(LION)
    gpu = run_gpu(inp)
    cu = inp["cu_seqlens"]
    for b in (11,):  # a sampled sequence: its y and dx depend on it alone
        s, e = int(cu[b]), int(cu[b + 1])
        sub = dict(inp, x=inp["x"][s:e], dy=inp["dy"][s:e], cu_seqlens=np.array([0, e - s], np.int32))
        y = ol.forward_full(*oracle_args(sub), inp["H"])
        g = ol.backward_full(*oracle_args(sub), sub["dy"], inp["H"])
        errs = {"y": rel_err(gpu["y"][s:e], y), "dx": rel_err(gpu["dx"][s:e], g["dx"])}
        print(f"\n[full size, sequence {b}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        assert max(errs.values()) <= TOL["bf16"], errs
    # y is linear in W_V (the attention weights do not depend on it), so
    # <W_V, dW_V> = <y, dy> for the whole batch.
    lhs = float(np.sum(inp["w_v"].astype(np.float64) * gpu["dw_v"]))
    rhs = float(np.sum(gpu["y"].astype(np.float64) * inp["dy"]))
    print(f"[full size] <W_V, dW_V> = {lhs:.6e}, <y, dy> = {rhs:.6e}", flush=True)
    assert abs(lhs - rhs) <= 2e-2 * max(abs(rhs), np.sqrt(np.sum(gpu["y"].astype(np.float64) ** 2)))
    for k in GRADS:
        assert np.all(np.isfinite(gpu[k])), k


# ------------------------------------------------------------ properties of the GPU path itself

def _small_bf16():
    return make_inputs(small_variant(LION, (300, 65, 1, 0, 200), d_model=128, num_heads=2, seed=55))


def test_f32_many_sequences():
    """More sequences than the schedule block has threads (256): the chunk table
    is built in several batches, with empty and single-token sequences among them."""
    rng = np.random.default_rng(60)
    lens = rng.integers(0, 30, 600)
    lens[rng.choice(600, 50, replace=False)] = 0
    lens[[5, 300, 599]] = (200, 1, 129)
    w = small_variant(LION, lens, d_model=64, num_heads=2, dtype="f32", seed=60)
    compare(make_inputs(w), label="f32 600 sequences")


def test_bitwise_deterministic():
    inp = _small_bf16()
    a, b = run_gpu(inp), run_gpu(inp)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_packed_sequences_are_isolated():
    """Changing one sequence's tokens leaves every other sequence's y and dx
    bitwise unchanged."""
    inp = _small_bf16()
    a = run_gpu(inp)
    cu = inp["cu_seqlens"]
    inp2 = dict(inp, x=inp["x"].copy())
    inp2["x"][cu[0]:cu[1]] = inp2["x"][cu[0]:cu[1]][::-1]
    b = run_gpu(inp2)
    keep = np.ones(inp["T"], bool)
    keep[cu[0]:cu[1]] = False
    for k in ("y", "dx"):
        assert np.array_equal(a[k][keep], b[k][keep]), k
        assert not np.array_equal(a[k][~keep], b[k][~keep]), k


def test_single_token_sequence_returns_v():
    """L = 1: the only attention weight is the token itself, so y = v."""
    inp = make_inputs(small_variant(LION, (1, 1, 1), d_model=64, num_heads=2, dtype="f32", seed=56))
    gpu = run_gpu(inp, backward=False)
    v = inp["x"].astype(np.float64) @ inp["w_v"].astype(np.float64)
    assert rel_err(gpu["y"], v) <= 1e-5


def test_no_tokens():
    inp = make_inputs(small_variant(LION, (0, 0), d_model=64, num_heads=2, seed=57))
    out = run_gpu(inp)
    assert out["y"].shape == (0, 128)
    for k in ("dw_q", "dw_k", "dw_v", "dw_lam", "db_lam"):
        assert np.all(out[k] == 0), k


# ------------------------------------------------------------ Lion-d and Lion-lit (the other two decays)

def run_gpu_decay(inp, decay, b):
    """decay "d": lambda^h = sigmoid(b[h]); "lit": lambda = 1. No w_lam."""
    d = to_dev(inp)
    H = inp["H"]
    bl = torch.from_numpy(b).float().to("cuda") if b is not None else None
    y, act = gl.forward(d["x"], d["cu"], d["w_q"], d["w_k"], d["w_v"], None, bl, H, decay=decay)
    g = gl.backward(d["x"], d["cu"], d["w_q"], d["w_k"], d["w_v"], None, bl, act, y, d["dy"], H, decay=decay)
    torch.cuda.synchronize()
    out = {"y": y}
    out.update(g)
    return {k: v.float().cpu().numpy() for k, v in out.items()}


def compare_decay(inp, decay, label, db_sum=False):
    """Lion-d is the oracle's selective form with w_lam = 0 (the logit is b_lam
    for every token: M_ij = lambda^|i-j|); Lion-lit is lambda = 1 (b_lam = +inf,
    M = 1). Compared: y, dx, dW_Q, dW_K, dW_V and, for Lion-d, db_lam."""
    H, dtype = inp["H"], inp["dtype"]
    b = np.random.default_rng(60).uniform(0.0, 4.0, size=H).astype(np.float32) if decay == "d" else None
    gpu = run_gpu_decay(inp, decay, b)
    ob = b if decay == "d" else np.full(H, np.inf, np.float32)
    args = [inp["x"], inp["cu_seqlens"], inp["w_q"], inp["w_k"], inp["w_v"], np.zeros_like(inp["w_lam"]), ob]
    errs = {"y": rel_err(gpu["y"], ol.forward_full(*args, H))}
    g = ol.backward_full(*args, inp["dy"], H)
    e, bounded = grad_errors(gpu, g, ("dx", "dw_q", "dw_k", "dw_v") + (("db_lam",) if decay == "d" else ()), db_sum)
    errs.update(e)
    bounded.update({"y": errs["y"]})
    print(f"\n[Lion-{decay} {dtype} {label}] T={inp['T']}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    assert set(gpu) == {"y", "dx", "dw_q", "dw_k", "dw_v"} | ({"db_lam"} if decay == "d" else set())
    bad = {k: v for k, v in bounded.items() if not v <= TOL[dtype]}
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["d", "lit"])
def test_fixed_and_no_decay_match_the_oracle(decay, dtype):
    w = small_variant(LION, (300, 65, 1, 130), d_model=96, num_heads=3, dtype=dtype, seed=59)
    compare_decay(make_inputs(w), decay, "short")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["d", "lit"])
def test_fixed_and_no_decay_many_chunks(decay, dtype):
    """Lion-d and Lion-lit over 18 and 71 chunks (every scan and suffix round).
    With one decay per head, db_lam = sum_t da_t over 5600 tokens cancels by a
    factor of about 350 here (printed as db_lam_cancel), so its bound is on the
    error relative to the summed terms; the plain error is printed beside it."""
    w = small_variant(LION, (1100, 4500, 7), d_model=128, num_heads=2, dtype=dtype, seed=71)
    compare_decay(make_inputs(w), decay, "18/71-chunk sequences", db_sum=decay == "d")
