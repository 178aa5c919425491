#!/usr/bin/env python3
"""GBLA forward+backward throughput on one MI355X.

One step = one gbla_forward + one gbla_backward (every stage of the layer's hot
path) over one synthetic batch of the long-history workload: 8 sequences x 8192
tokens, d_model 512, 8 heads of 64, bf16 activations and weights with fp32
accumulation, 10% repeated rows, gate bias +1. Inputs are resident in HBM
before the timed region; x and dy rotate over three buffer sets (> 256 MB) so
the 256 MB Infinity Cache does not serve a step from the previous step's data.

Prints ONE JSON line: tokens/s (value), the roofline of the dominant stage
measured live with the library's HIP events on the launch stream, recorded in
the timed region around that stage only (a pass before it, with events around
every stage, gives stage_ms_per_step and picks the dominant stage), and the
float64 CPU oracle timed on a bounded sample of the same workload.
The same line carries secondary measurements: the GBLA layer on the 32 x 1024
(d 256) and ragged 256-sequence workloads ("gbla_B32_L1024_d256",
"gbla_ragged_N256_d512"), its forward-only latency at batch 8 and L = 8192 and
32768 beside the pages' H100 figures ("forward_latency"), the main workload
with the softmax-over-the-sequence key gate under "gbla_softmax" and with the
gated RMSNorm output (Eq. (7)) under "gbla_gated_rmsnorm", and the LION layers
(16 x 4096 tokens, d_model 512, 8 heads of 64, 64-token chunks, bf16) under
"lion_s", "lion_d" and "lion_lit" (selective, fixed per-head and no decay).

--copy-calibration instead times a plain device-to-device copy of a known size
(for scaling the FETCH_SIZE / WRITE_SIZE counters of rocprofv3 to bytes).
--hbm-ceiling instead measures the practical HBM rate of a streaming copy (the
context for the bandwidth-bound kernels' fraction of the 8 TB/s peak).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA, TFLOP/s
WORKLOAD = "gbla_bf16_B8_L8192_d512"


def stage_work(stage, T, N, d, H, dh, esz, nsplit=1):
    """Algorithmic work of one launch of a stage: ("mfma", flops) or ("hbm", bytes).
    Bytes count each compulsory operand once; flops count the dense contraction."""
    D = H * dh
    P3 = 3 * D + H
    table = {
        "proj_fwd": ("mfma", 2.0 * T * d * 3 * D),
        "proj_recompute": ("mfma", 2.0 * T * d * 3 * D),
        "conv_fwd": ("hbm", 2.0 * T * d * esz + 4.0 * T * H),
        "gemm_dx": ("mfma", 2.0 * T * P3 * d),
        "gemm_dw": ("mfma", 2.0 * T * d * P3),
        "state_partial": ("hbm", 2.0 * T * D * esz),
        "readout": ("hbm", 2.0 * T * D * esz),
        "bwd_dstate": ("hbm", 3.0 * T * D * esz),
        "bwd_token": ("hbm", 4.0 * T * D * esz + 4.0 * T * H + esz * T * H),
        "conv_bwd": ("hbm", 3.0 * T * d * esz),
    }
    return table.get(stage)


def layer_bytes_per_token(d, D, esz):
    """Compulsory HBM bytes per token of one fwd+bwd: x read twice-free (once per
    pass), y written, dy read, dx written (weights and states are negligible)."""
    return esz * (d + D) + esz * (d + D + d)


def traffic_for(stage):
    """HBM bytes per launch of the stage's kernel from the committed rocprofv3
    counter summary (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE scaled by
    the factors measured on a copy of known size), or None if there is none or
    any source file of the kernel changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(stage)
    except Exception:
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        full = os.path.join(ROOT, src)
        if not os.path.exists(full):
            return None
        h.update(open(full, "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["bytes_per_launch"]


def cpu_baseline(inp, sample_seqs, repeats=3):
    """Time the float64 oracle (fwd+bwd) on the first `sample_seqs` sequences,
    `repeats` times; the median run gives the rate."""
    import numpy as np
    from oracle import gbla as og
    host_cores = len(os.sched_getaffinity(0))
    # the oracle's BLAS threads: the host cores this process may run on, capped
    # by OMP_NUM_THREADS where the environment sets it (the GPU host's CPU share)
    want = host_cores
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        want = max(1, min(want, int(os.environ["OMP_NUM_THREADS"])))
    limiter, blas = None, "unknown"
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=want, user_api="blas")
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '?')} threads)"
                         for i in info) or "unknown"
    except Exception:
        threads = 1
    cu = inp["cu_seqlens"]
    S = min(sample_seqs, inp["N"])
    T = int(cu[S])
    sub = dict(inp, x=inp["x"][:T], dy=inp["dy"][:T], cu_seqlens=cu[:S + 1].copy())
    args = [sub[k] for k in ("x", "cu_seqlens", "conv_w", "w_q", "w_k", "w_v", "w_g", "b_g")]
    runs = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        og.forward(*args, inp["H"])
        og.backward(*args, sub["dy"], inp["H"])
        runs.append(time.perf_counter() - t0)
    dt = sorted(runs)[len(runs) // 2]
    if limiter is not None:
        limiter.restore_original_limits()
    del np
    return {"value": T / dt, "unit": "tokens/s", "cores": int(threads), "host_cores": host_cores, "blas": blas,
            "kind": "oracle",
            "sample": f"float64 numpy oracle forward+backward on the first {S} of {inp['N']} sequences "
                      f"({T} tokens) of the same batch, median of {repeats} runs "
                      f"({', '.join(f'{r:.1f}' for r in runs)} s)"}


def timed_passes(gb, torch, step, steps, warmup, stage_filter):
    """Warm up, then (1) an untimed pass with every stage's events for the
    breakdown, (2) the timed region: `steps` steps bracketed by synchronize,
    with events recorded only around the stages stage_filter(breakdown) picks
    (each recorded event costs device time). Returns (elapsed seconds,
    breakdown {stage: (ms, launches)} per pass-1 step, timed-region stages)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    nb = max(1, min(steps, 10))
    gb.profile_begin(64 * nb)
    for i in range(nb):
        step(i)
    torch.cuda.synchronize()
    br = gb.profile_end()
    breakdown = {k: (v[0] / nb, v[1] / nb) for k, v in br.items()}
    sel = stage_filter(breakdown)
    gb.profile_begin(64 * max(1, steps), stages=sel)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    timed = gb.profile_end()
    return t1 - t0, breakdown, timed


def copy_calibration(mib=1024, reps=3):
    """Copy `mib` MiB device to device `reps` times; the copy kernel reads and
    writes exactly mib MiB per launch."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.randn(n, device="cuda:0").to(torch.bfloat16)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n * 2, "bytes_written_per_launch": n * 2,
                                           "launches": reps, "gb_per_s": round(2 * n * 2 / dt / 1e9, 1)}}),
          flush=True)


def hbm_ceiling(mib=64, reps=10):
    """Rate of a device-to-device copy of `mib` MiB (bytes read + written over
    the copy's time, HIP events on its stream). "cold": each timed copy follows
    a read-only sum over a 1 GiB buffer, so the 256 MB last-level cache holds
    none of the copy's operands (a write sweep would leave dirty lines whose
    write-back the copy would pay for); "warm": the same copy repeated at once,
    its operands cache-resident. Medians over `reps` pairs."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.randn(n, device="cuda:0").to(torch.bfloat16)
    dst = torch.empty_like(src)
    sweep = torch.ones((1 << 30) // 4, device="cuda:0")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    cold, warm = [], []
    for i in range(reps + 2):
        torch.sum(sweep)
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        ev[2].record()
        dst.copy_(src)
        ev[3].record()
        torch.cuda.synchronize()
        if i >= 2:
            cold.append(ev[0].elapsed_time(ev[1]) * 1e-3)
            warm.append(ev[2].elapsed_time(ev[3]) * 1e-3)
    moved = 2 * n * 2
    med = lambda v: sorted(v)[len(v) // 2]
    print(json.dumps({"hbm_ceiling": {
        "copy_bytes_read_plus_written": moved, "pairs": reps,
        "cold_tb_per_s": round(moved / med(cold) / 1e12, 3), "warm_tb_per_s": round(moved / med(warm) / 1e12, 3),
        "cold_us": round(med(cold) * 1e6, 2), "warm_us": round(med(warm) * 1e6, 2),
        "flush": "read-only sum over a 1 GiB buffer before each cold copy", "peak_tb_per_s": 8.0}}), flush=True)


def gbla_setup(torch, gb, gate, gated_output=False, workload=WORKLOAD, n_sets=3):
    """Device buffers and the step function of a GBLA workload (x and dy
    rotate over n_sets buffer sets); gated_output adds the gated RMSNorm output
    (W_R, gamma). Also returns fwd(i), the forward pass alone."""
    import numpy as np

    from bidirectional_linear_attention_amd.synthetic import WORKLOADS, make_inputs, make_output_gate

    w = WORKLOADS[workload]
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    esz = 2 if w.dtype == "bf16" else 4

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt).contiguous()

    T, N, d, H, dh = inp["T"], inp["N"], inp["d"], inp["H"], inp["dh"]
    D = H * dh
    cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
    conv_w, w_q, w_k, w_v, w_g = (t(inp[k]) for k in ("conv_w", "w_q", "w_k", "w_v", "w_g"))
    b_g = torch.from_numpy(inp["b_g"]).float().to(dev)
    xs = [t(inp["x"]) for _ in range(n_sets)]
    dys = [t(inp["dy"]) for _ in range(n_sets)]
    p = gb.problem(N, T, d, H, dh, dt, gate, gated_output)
    og = dict(w_r=None, gamma=None, dw_r=None, dgamma=None)
    if gated_output:
        o = make_output_gate(w)
        og = dict(w_r=t(o["w_r"]), gamma=torch.from_numpy(o["gamma"]).float().to(dev),
                  dw_r=torch.empty((d, D), dtype=torch.float32, device=dev),
                  dgamma=torch.empty((dh,), dtype=torch.float32, device=dev))
    y = torch.empty((T, D), dtype=dt, device=dev)
    saved = torch.empty(gb.saved_size(p) // 4, dtype=torch.float32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dx = torch.empty((T, d), dtype=dt, device=dev)
    dconv = torch.empty((d, 4), **f32)
    dwq, dwk, dwv = (torch.empty((d, D), **f32) for _ in range(3))
    dwg, dbg = torch.empty((H, d), **f32), torch.empty((H,), **f32)
    ws = torch.empty(max(gb.workspace_size(p, False), gb.workspace_size(p, True)), dtype=torch.uint8, device=dev)
    act = torch.empty(gb.activation_size(p), dtype=torch.uint8, device=dev)

    def fwd(i):
        gb.gbla_forward(p, xs[i % n_sets], cu, conv_w, w_q, w_k, w_v, w_g, b_g, y, saved, act, ws, w_r=og["w_r"],
                        gamma=og["gamma"])

    def step(i):
        fwd(i)
        gb.gbla_backward(p, xs[i % n_sets], cu, conv_w, w_q, w_k, w_v, w_g, b_g, saved, act, dys[i % n_sets], dx,
                         dconv, dwq, dwk, dwv, dwg, dbg, ws, **og)

    return dict(w=w, inp=inp, step=step, fwd=fwd, T=T, N=N, d=d, H=H, dh=dh, esz=esz)


def gbla_workload_leg(steps, warmup, workload):
    """GBLA forward+backward (sigmoid key gate, plain output) on another workload
    of the recipe table: tokens/s and stage times."""
    import torch

    import bidirectional_linear_attention_amd as gb

    g = gbla_setup(torch, gb, "sigmoid", workload=workload)
    elapsed, breakdown, _ = timed_passes(gb, torch, g["step"], steps, warmup, lambda br: [])
    T = g["T"]
    return {"workload": workload, "sequences": g["N"], "tokens_per_step": T, "steps": steps, "warmup": warmup,
            "tokens_per_s": round(T * steps / elapsed, 1), "ms_per_step": round(1e3 * elapsed / steps, 4),
            "stage_ms_per_step": {k: round(v[0], 4) for k, v in sorted(breakdown.items(), key=lambda kv: -kv[1][0])}}


# forward-only single-layer latency of GBLA on an H100 in the GBLA page's
# benchmark section (Table 5: batch 8, mean of 10 runs, precision and layer
# boundary not stated); context for the forward latency legs, not a target
PAGES_FORWARD_MS = {"gbla_bf16_B8_L8192_d512": 2.2, "gbla_bf16_B8_L32768_d512": 8.2}


def forward_latency_leg(workload, runs=10, warmup=3):
    """Forward-only latency of one layer call (batch 8, L = 8192 or 32768): the
    mean of `runs` calls, each bracketed by synchronize, as the pages time it."""
    import torch

    import bidirectional_linear_attention_amd as gb

    g = gbla_setup(torch, gb, "sigmoid", workload=workload, n_sets=2)
    for i in range(warmup):
        g["fwd"](i)
    torch.cuda.synchronize()
    times = []
    for i in range(runs):
        t0 = time.perf_counter()
        g["fwd"](i)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    ms = 1e3 * sum(times) / len(times)
    return {"workload": workload, "tokens": g["T"], "forward_ms_mean": round(ms, 4), "runs": runs,
            "forward_tokens_per_s": round(g["T"] / (ms / 1e3), 1),
            "pages_h100_forward_ms": PAGES_FORWARD_MS.get(workload),
            "note": "context only: the pages' figure is another machine, precision and layer boundary unstated"}


def gbla_variant_leg(steps, warmup, gate="sigmoid", gated_output=False):
    """The same GBLA workload with the softmax-over-the-sequence key gate or
    the gated RMSNorm output."""
    import torch

    import bidirectional_linear_attention_amd as gb

    g = gbla_setup(torch, gb, gate, gated_output)
    elapsed, breakdown, _ = timed_passes(gb, torch, g["step"], steps, warmup, lambda br: [])
    T = g["T"]
    return {"workload": g["w"].name, "key_gate": gate + (" over the sequence" if gate == "softmax" else ""),
            "output": "gated RMSNorm (Eq. 7)" if gated_output else "plain", "tokens_per_step": T, "steps": steps,
            "warmup": warmup, "tokens_per_s": round(T * steps / elapsed, 1),
            "ms_per_step": round(1e3 * elapsed / steps, 4),
            "stage_ms_per_step": {k: round(v[0], 4) for k, v in sorted(breakdown.items(), key=lambda kv: -kv[1][0])}}


def lion_leg(steps, warmup, decay="s"):
    """LION forward+backward on the 16 x 4096 workload: tokens/s and stage times.
    decay "s" (Lion-s), "d" (Lion-d: the workload's b_lam as the per-head logit)
    or "lit" (Lion-lit)."""
    import numpy as np
    import torch

    from bidirectional_linear_attention_amd import lion as gl
    from bidirectional_linear_attention_amd.synthetic import WORKLOADS, make_inputs

    w = WORKLOADS["lion_s_bf16_B16_L4096_d512"]
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt).contiguous()

    T, N, d, H, dh = inp["T"], inp["N"], inp["d"], inp["H"], inp["dh"]
    D = H * dh
    cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
    w_q, w_k, w_v, w_lam = (t(inp[k]) for k in ("w_q", "w_k", "w_v", "w_lam"))
    b_lam = torch.from_numpy(inp["b_lam"]).float().to(dev)
    n_sets = 3
    xs = [t(inp["x"]) for _ in range(n_sets)]
    dys = [t(inp["dy"]) for _ in range(n_sets)]
    p = gl.problem(N, T, d, H, dh, dt, decay)
    f32 = dict(dtype=torch.float32, device=dev)
    y = torch.empty((T, D), dtype=dt, device=dev)
    dx = torch.empty((T, d), dtype=dt, device=dev)
    dwq, dwk, dwv = (torch.empty((d, D), **f32) for _ in range(3))
    dwl, dbl = torch.empty((H, d), **f32), torch.empty((H,), **f32)
    if decay != "s":
        w_lam, dwl = None, None
    if decay == "lit":
        b_lam, dbl = None, None
    ws = torch.empty(max(gl.workspace_size(p, False), gl.workspace_size(p, True)), dtype=torch.uint8, device=dev)
    act = torch.empty(gl.activation_size(p), dtype=torch.uint8, device=dev)

    def step(i):
        x, dy = xs[i % n_sets], dys[i % n_sets]
        gl.lion_forward(p, x, cu, w_q, w_k, w_v, w_lam, b_lam, y, act, ws)
        gl.lion_backward(p, x, cu, w_q, w_k, w_v, w_lam, b_lam, act, y, dy, dx, dwq, dwk, dwv, dwl, dbl, ws)

    import bidirectional_linear_attention_amd as gb
    elapsed, breakdown, _ = timed_passes(gb, torch, step, steps, warmup, lambda br: [])
    return {"workload": w.name, "decay": {"s": "Lion-s", "d": "Lion-d", "lit": "Lion-lit"}[decay],
            "tokens_per_step": T, "steps": steps, "warmup": warmup,
            "tokens_per_s": round(T * steps / elapsed, 1), "ms_per_step": round(1e3 * elapsed / steps, 4),
            "stage_ms_per_step": {k: round(v[0], 4) for k, v in sorted(breakdown.items(), key=lambda kv: -kv[1][0])}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-sample-seqs", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lion-steps", type=int, default=10,
                    help="steps of each secondary leg (softmax-gate GBLA, Lion-s/d/lit) after the main run (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--hbm-ceiling", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the GBLA/LION path here runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is designed but not implemented)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.hbm_ceiling:
        hbm_ceiling()
        return

    import torch

    import bidirectional_linear_attention_amd as gb

    g = gbla_setup(torch, gb, "sigmoid")
    w, inp, step = g["w"], g["inp"], g["step"]
    T, N, d, H, dh, esz = (g[k] for k in ("T", "N", "d", "H", "dh", "esz"))
    D = H * dh

    def dominant(br):
        timed = {k: v for k, v in br.items() if stage_work(k, T, N, d, H, dh, esz)}
        return [max(timed, key=lambda k: timed[k][0])]

    elapsed, breakdown, timed = timed_passes(gb, torch, step, args.steps, args.warmup, dominant)
    ms_per_step = 1e3 * elapsed / args.steps
    tok_s = T * args.steps / elapsed

    # roofline of the dominant stage from its events inside the timed region
    dom = dominant(breakdown)[0]
    bound, work = stage_work(dom, T, N, d, H, dh, esz)
    dom_ms, dom_launches = timed[dom]
    avg_s = dom_ms / dom_launches / 1e3
    if bound == "mfma":
        achieved, peak, unit = work / avg_s / 1e12, MFMA_PEAK_TFLOPS[w.dtype], "TFLOP/s"
    else:
        achieved, peak, unit = work / avg_s / 1e9, HBM_PEAK_GBS, "GB/s"
    roof = {"bound": bound, "kernel": dom, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic_for(dom),
            "avg_launch_us": round(avg_s * 1e6, 2)}
    per_step = {k: v[0] for k, v in breakdown.items()}

    bpt = layer_bytes_per_token(d, D, esz)
    out = {
        "metric": "GBLA fwd+bwd tokens/s at L=8192,H=8,d_h=64 bf16; % of HBM roofline",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "global_batch": N, "seq_len": T // N, "d_model": d, "num_heads": H,
                   "head_dim": dh, "tokens_per_step": T, "parallelism": "none (1 GPU)"},
        "hbm_roofline_frac_layer": round(bpt * tok_s / (HBM_PEAK_GBS * 1e9), 4),
        "roofline": roof,
        "stage_ms_per_step": {k: round(v, 4) for k, v in sorted(per_step.items(), key=lambda kv: -kv[1])},
    }
    if args.lion_steps > 0:
        del g, step
        torch.cuda.empty_cache()
        out["gbla_B32_L1024_d256"] = gbla_workload_leg(args.lion_steps, min(args.warmup, 3),
                                                        "gbla_bf16_B32_L1024_d256")
        torch.cuda.empty_cache()
        out["gbla_ragged_N256_d512"] = gbla_workload_leg(args.lion_steps, min(args.warmup, 3),
                                                          "gbla_bf16_ragged_N256_d512")
        torch.cuda.empty_cache()
        out["forward_latency"] = [forward_latency_leg(wl) for wl in ("gbla_bf16_B8_L8192_d512",
                                                                      "gbla_bf16_B8_L32768_d512")]
        torch.cuda.empty_cache()
        out["gbla_softmax"] = gbla_variant_leg(args.lion_steps, min(args.warmup, 3), gate="softmax")
        torch.cuda.empty_cache()
        out["gbla_gated_rmsnorm"] = gbla_variant_leg(args.lion_steps, min(args.warmup, 3), gated_output=True)
        torch.cuda.empty_cache()
        out["lion_s"] = lion_leg(args.lion_steps, min(args.warmup, 3))
        for dec in ("d", "lit"):
            out["lion_" + dec] = lion_leg(args.lion_steps, min(args.warmup, 3), dec)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_seqs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
