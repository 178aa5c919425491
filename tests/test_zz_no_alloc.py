"""The allocation-free forward (include/gbla.h: gbla_forward_noalloc) against
gbla_forward, through the C ABI: the same kernels on the same inputs, so y and
the saved states must be bitwise equal. Two calls in a row, the second on a
smaller problem (the static scratch keeps the first call's contents, which the
second must not read), with and without an activation cache, and the oracle's
float64 forward as a check of the first call."""
import numpy as np
import pytest
import torch

import bidirectional_linear_attention_amd as gb
from bidirectional_linear_attention_amd import _lib
from bidirectional_linear_attention_amd.synthetic import WORKLOADS, make_inputs, small_variant
from oracle import gbla as og

pytestmark = pytest.mark.gpu

BASE = WORKLOADS["gbla_bf16_B8_L8192_d512"]


def _dev(inp):
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt).contiguous()

    return dict(x=t(inp["x"]), cu=torch.from_numpy(inp["cu_seqlens"]).to("cuda"), conv_w=t(inp["conv_w"]),
                w_q=t(inp["w_q"]), w_k=t(inp["w_k"]), w_v=t(inp["w_v"]), w_g=t(inp["w_g"]),
                b_g=torch.from_numpy(inp["b_g"]).float().to("cuda"))


def _run(inp, noalloc, with_act):
    d = _dev(inp)
    p = gb.problem(inp["N"], inp["T"], inp["d"], inp["H"], inp["dh"], d["x"].dtype)
    # zero-filled, so that the cache's alignment padding (written by neither call) compares equal
    y = torch.zeros((inp["T"], inp["H"] * inp["dh"]), dtype=d["x"].dtype, device="cuda")
    saved = torch.zeros(gb.saved_size(p) // 4, dtype=torch.float32, device="cuda")
    act = torch.zeros(gb.activation_size(p), dtype=torch.uint8, device="cuda") if with_act else None
    args = (p, d["x"], d["cu"], d["conv_w"], d["w_q"], d["w_k"], d["w_v"], d["w_g"], d["b_g"], y, saved, act)
    if noalloc:
        gb.gbla_forward_noalloc(*args)
    else:
        ws = torch.empty(gb.workspace_size(p, False), dtype=torch.uint8, device="cuda")
        gb.gbla_forward(*args, ws)
    torch.cuda.synchronize()
    out = {"y": y.float().cpu().numpy(), "saved": saved.cpu().numpy()}
    if with_act:
        out["act"] = act.cpu().numpy()
    return out


@pytest.mark.parametrize("with_act", [True, False])
def test_noalloc_forward_equals_forward_on_two_calls(with_act):
    big = make_inputs(small_variant(BASE, (2000, 700, 1, 1500), d_model=256, num_heads=4, seed=81))
    small = make_inputs(small_variant(BASE, (300, 45), d_model=128, num_heads=2, seed=82))
    for i, inp in enumerate((big, small)):
        ref = _run(inp, noalloc=False, with_act=with_act)
        got = _run(inp, noalloc=True, with_act=with_act)
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (i, k)
        y = og.forward(*[inp[k] for k in ("x", "cu_seqlens", "conv_w", "w_q", "w_k", "w_v", "w_g", "b_g")],
                       inp["H"])[0]
        err = float(np.max(np.abs(got["y"] - y)) / np.max(np.abs(y)))
        print(f"\n[noalloc call {i}, act={with_act}] T={inp['T']} d={inp['d']} H={inp['H']}: "
              f"bitwise equal to gbla_forward; y vs oracle {err:.2e}", flush=True)
        assert err <= 2e-2


def test_noalloc_forward_rejects_a_problem_beyond_its_scratch():
    """Without an activation cache the activations need scratch too: a problem
    whose workspace exceeds the static array is refused before any launch."""
    T = 200_000
    p = gb.problem(1, T, 512, 8, 64, torch.bfloat16)
    assert gb.workspace_size(p, False) > _lib.STATIC_SCRATCH_BYTES
    x = torch.zeros((T, 512), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    w = torch.zeros((512, 512), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, 512), dtype=torch.bfloat16, device="cuda")
    saved = torch.empty(gb.saved_size(p) // 4, dtype=torch.float32, device="cuda")
    with pytest.raises(gb.GblaError, match="SCRATCH_LIMIT"):
        gb.gbla_forward_noalloc(p, x, cu, torch.zeros((512, 4), dtype=torch.bfloat16, device="cuda"), w, w, w,
                                torch.zeros((8, 512), dtype=torch.bfloat16, device="cuda"),
                                torch.zeros(8, dtype=torch.float32, device="cuda"), y, saved, None)


def test_noalloc_forward_replays_under_graph_capture():
    """The allocation-free forward captured into a graph (torch.cuda.graph)
    and replayed three times, new inputs copied into the captured buffers
    before each replay; every replay is compared bitwise with an eager call of
    the same entry point on the same inputs, made between the replays."""
    w = small_variant(BASE, (1200, 333, 900), d_model=256, num_heads=4, seed=83)
    inps = [make_inputs(w, seed=83 + i) for i in range(3)]
    bufs = _dev(inps[0])
    p = gb.problem(inps[0]["N"], inps[0]["T"], inps[0]["d"], inps[0]["H"], inps[0]["dh"], bufs["x"].dtype)
    y = torch.zeros((p.total_tokens, p.num_heads * p.head_dim), dtype=bufs["x"].dtype, device="cuda")
    saved = torch.zeros(gb.saved_size(p) // 4, dtype=torch.float32, device="cuda")
    args = (p, bufs["x"], bufs["cu"], bufs["conv_w"], bufs["w_q"], bufs["w_k"], bufs["w_v"], bufs["w_g"],
            bufs["b_g"], y, saved, None)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call first, off the capture
        gb.gbla_forward_noalloc(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gb.gbla_forward_noalloc(*args)
    n_saved = p.num_seqs * p.num_heads * (p.head_dim * p.head_dim + p.head_dim)
    for i, inp in enumerate(inps):
        new = _dev(inp)
        for k in ("x", "conv_w", "w_q", "w_k", "w_v", "w_g", "b_g"):
            bufs[k].copy_(new[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_y, got_s = y.float().cpu().numpy(), saved.cpu().numpy()[:n_saved]
        ref = _run(inp, noalloc=True, with_act=False)
        assert np.array_equal(got_y, ref["y"]), i
        assert np.array_equal(got_s, ref["saved"][:n_saved]), i
        print(f"\n[graph replay {i}] T={inp['T']} d={inp['d']} H={inp['H']}: bitwise equal to the eager call",
              flush=True)
