#!/usr/bin/env python3
"""MoE-layer tokens/s on one MI355X, with the roofline of the dominant kernel.

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill|skewed|tiny|stack|decode_fp8|backward]

One step is one pass of the whole layer (router -> permute -> gate/up + SwiGLU ->
down -> combine) over one batch of synthetic tokens already resident in HBM.

Phase A times K steps of moe_layer_forward between device synchronisations (the
reported value and ms_per_step, the mean over that window), with a HIP event
recorded on the launch stream before every step and after the last, which gives
the median per-step time too.  Phase B runs K more steps through
moe_layer_forward_timed, the same launch sequence with HIP events recorded on
the stream between its five stages, which gives each stage's average duration
inside the layer (the down projection with its K split and tail pass, as the
layer runs it) and the dominant kernel's duration for the roofline figure.  The
CPU oracle is then timed on a bounded sample of the same workload.

The default run measures the decode workload (the headline value) and then the
prefill workload, reported as the "prefill" block of the same line (the MFMA
half of the metric); --no-prefill leaves that block out.

decode_fp8 is the decode workload with its expert weights quantized to FP8
(E4M3, one scale per row) on the device before any timing; its stages are
timed through the FP8 entry points, which are the FP8 layer's own kernels.
backward times moe_layer_backward (all gradients of the layer) on the prefill
workload's inputs with a seeded upstream gradient; its roofline covers the
whole pass.  stack runs 32 pre-norm MoE blocks (h <- h + MoE(RMSNorm(h)),
independent weights per layer, ~90 GB resident) over 8192 tokens: one step is
the whole stack, and the roofline is that of the gate/up kernel averaged over
the layers.

Prints one JSON line.  Only one GPU is used; --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 MI355X + % of HBM (decode) / MFMA (prefill) roofline"
WORKLOADS = {"tiny": 0, "decode": 1, "prefill": 2, "skewed": 3, "stack": 4, "decode_fp8": 1, "backward": 2}
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sparse_moe_transformer_way_amd", "csrc")
# source file of each kernel the roofline can name
KERNEL_SRC = {"gate_up_stream": "grouped_gemm.hip", "gate_up_tiled": "tiled_gemm.hip",
              "gate_up_f32": "grouped_gemm.hip", "gate_up_stream_fp8": "grouped_gemm.hip"}
STAGES = ["router_topk", "permute", "expert_gate_up", "expert_down", "combine"]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="minimum host time spent timing the CPU oracle per workload (0 skips it)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode only: leave out the prefill block of the default run")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--vs-library", action="store_true",
                    help="only compare the tiled expert projections with hipBLASLt (torch.bmm) on the "
                         "same grouped shapes, with exactly balanced routing")
    return ap.parse_args()


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summary, or None when there is none or the kernel source changed since."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path) or kernel not in KERNEL_SRC:
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    h = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != source_digest(os.path.join(CSRC, KERNEL_SRC[kernel])):
        return None
    return float(m.group(1))


def calibrate_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "copies": 5}))


def vs_library(args):
    """The two expert projections at prefill and stack sizes (T = 4096, 8192; d = 4096,
    F = 14336, 8 experts, top-2) with exactly balanced routing, T*K/8 rows per expert:
    moe_expert_gate_up / moe_expert_down (tile 256) against hipBLASLt's batched GEMM
    (torch.bmm, one batch per expert, contiguous operands) on the same shapes.  The
    library GEMMs compute less: no gather of x rows, no SwiGLU (gate/up writes both
    2F-wide products), no ragged segments.  The chip's clock ramps up over the first
    tens of milliseconds of load, so each kernel first runs for half a second, and the
    four kernels are then timed in three interleaved rounds (median over all calls).
    Prints one JSON line."""
    import torch
    import sparse_moe_transformer_way_amd as moe

    dev = torch.device("cuda")
    d, F, n, K = 4096, 14336, 8, 2
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def warm(fn, seconds=0.5):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()

    def timed(fn):
        ev = events(args.steps + 1, stream)
        torch.cuda.synchronize()
        for s in range(args.steps):
            ev[s].record(stream)
            fn()
        ev[args.steps].record(stream)
        torch.cuda.synchronize()
        return [ev[s].elapsed_time(ev[s + 1]) for s in range(args.steps)]

    def randn(*shape):
        return (torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)

    rows = []
    for T in (4096, 8192):
        M = T * K // n
        desc = moe.make_desc(d, F, n, K, dtype=torch.bfloat16)
        x = randn(T, d)
        w1, w3, w2 = randn(n, F, d), randn(n, F, d), randn(n, d, F)
        counts = torch.full((n,), M, dtype=torch.int32, device=dev)
        offsets = torch.arange(0, n * M + 1, M, dtype=torch.int32, device=dev)
        # expert e takes the assignments t*K + k with (t*K + k) % n == e, in token order
        # (segments of M rows, a multiple of the tile: no padding rows inside them)
        P = moe.moe_max_permuted_rows(desc, T, 256)
        a = torch.arange(T * K, device=dev, dtype=torch.int32)
        row_src = torch.full((P,), -1, dtype=torch.int32, device=dev)
        row_src[:n * M] = torch.cat([a[a % n == e] for e in range(n)])
        h = torch.empty((P, F), dtype=torch.bfloat16, device=dev)
        y_perm = torch.empty((P, d), dtype=torch.float32, device=dev)
        xe = x[(row_src[:n * M] // K).long()].view(n, M, d).contiguous()
        w13t = torch.cat([w1, w3], dim=1).transpose(1, 2).contiguous()  # [n, d, 2F]
        w2t = w2.transpose(1, 2).contiguous()                            # [n, F, d]
        he = randn(n, M, F)
        fns = {
            "ours_gate_up": lambda: moe.moe_expert_gate_up(desc, T, 256, x, row_src, counts, offsets, w1, w3, h,
                                                           stream=stream),
            "ours_down": lambda: moe.moe_expert_down(desc, T, 256, h, counts, offsets, w2, y_perm, stream=stream),
            "lib_gate_up": lambda: torch.bmm(xe, w13t),
            "lib_down": lambda: torch.bmm(he, w2t),
        }
        for fn in fns.values():
            warm(fn)
        times = {k: [] for k in fns}
        for _ in range(3):
            for k, fn in fns.items():
                times[k] += timed(fn)
        med = {k: statistics.median(v) for k, v in times.items()}
        for name, flop in (("gate_up", 4.0 * n * M * d * F), ("down", 2.0 * n * M * F * d)):
            ours, lib = med["ours_" + name], med["lib_" + name]
            rows.append({"T": T, "rows_per_expert": M, "projection": name,
                         "ours_ms": round(ours, 4), "hipblaslt_bmm_ms": round(lib, 4),
                         "ours_mfma_frac": round(flop / ours / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "hipblaslt_mfma_frac": round(flop / lib / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)})
        del fns, x, w1, w3, w2, h, y_perm, xe, w13t, w2t, he
        torch.cuda.empty_cache()
    print(json.dumps({"comparison": "tiled expert projections vs hipBLASLt batched GEMM (torch.bmm), "
                      "balanced routing, median of per-call HIP events over three interleaved rounds",
                      "steps_per_round": args.steps, "rows": rows}), flush=True)


def host_facts() -> dict:
    """The host the CPU oracle runs on: logical CPUs, those this process may use,
    the CPU model and the BLAS thread count."""
    from threadpoolctl import threadpool_info
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": model,
            "blas_threads": blas}


def cpu_baseline(inp, seconds: float, rows_cap: int):
    """The oracle, as it stands, on a bounded sample of the workload's tokens."""
    import numpy as np
    import oracle

    xn, wgn, w1n, w3n, w2n = inp.numpy_f32()
    T = xn.shape[0]
    rows = np.arange(min(T, rows_cap))
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(xn[rows], wgn, w1n, w3n, w2n)
        done += rows.size
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    host = host_facts()
    return {"value": done / el, "unit": "tokens/s", "cores": host["blas_threads"], "kind": "oracle",
            "sample": f"the first {rows.size} of {T} tokens per call (dense fp32, all {wgn.shape[1]} experts), "
                      f"{done // rows.size} calls in {el:.1f} s",
            "host": host}


def events(n, stream):
    """n timing events, each recorded once so that its HIP handle exists."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record(stream)
    return ev


def run_layer(args, wl: int, fp8: bool, cpu_seconds: float) -> dict:
    """Measure one single-layer workload; returns the JSON object of its line."""
    import torch
    import moe_inputs as mi
    import sparse_moe_transformer_way_amd as moe

    spec = mi.WORKLOADS[wl]
    inp = mi.make_workload(wl, seed=args.seed)
    T, d, F, n, K = inp.T, inp.d, inp.F, inp.n, inp.K
    dt = torch.float32 if inp.dtype == "f32" else torch.bfloat16
    dev = torch.device("cuda")
    x, wg, w1, w3, w2 = (t.to(dev) for t in (inp.x, inp.wg, inp.w1, inp.w3, inp.w2))
    wl_name = spec["name"] + ("_fp8w" if fp8 else "")
    if fp8:
        # weights quantized once on the device, before any timing
        (q1, s1), (q3, s3), (q2, s2) = (moe.moe_quantize_fp8(w) for w in (w1, w3, w2))
        del w1, w3, w2
        torch.cuda.synchronize()
    desc = moe.make_desc(d, F, n, K, dtype=dt, weight_dtype=torch.float8_e4m3fn if fp8 else None)
    tile_m = moe.moe_default_tile_m(desc, T)
    P = moe.moe_max_permuted_rows(desc, T, tile_m)

    # outputs and scratch, allocated before any timing
    y = torch.empty((T, d), dtype=dt, device=dev)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    counts = torch.empty(n, dtype=torch.int32, device=dev)
    ws = torch.empty(moe.moe_workspace_size(desc, T, 0), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def layer_step():
        if fp8:
            moe.moe_layer_forward_fp8(desc, x, wg, q1, s1, q3, s3, q2, s2, y=y, topk_idx_out=idx,
                                      topk_gate_out=gate, counts_out=counts, workspace=ws, stream=stream)
        else:
            moe.moe_layer_forward(desc, x, wg, w1, w3, w2, y=y, topk_idx_out=idx, topk_gate_out=gate,
                                  counts_out=counts, workspace=ws, stream=stream)

    if fp8:
        # the FP8 layer's own kernels, one entry point per stage (no K split at tile 16)
        offsets = torch.empty(n + 1, dtype=torch.int32, device=dev)
        row_src = torch.empty(P, dtype=torch.int32, device=dev)
        row_of = torch.empty((T, K), dtype=torch.int32, device=dev)
        h = torch.empty((P, F), dtype=dt, device=dev)
        y_perm = torch.empty((P, d), dtype=torch.float32, device=dev)

        def staged_step(ev):
            ev[0].record(stream)
            moe.moe_router_topk(desc, x, wg, idx, gate, stream=stream)
            ev[1].record(stream)
            moe.moe_permute(desc, idx, tile_m, counts, offsets, row_src, row_of, stream=stream)
            ev[2].record(stream)
            moe.moe_expert_gate_up_fp8(desc, T, x, row_src, counts, offsets, q1, s1, q3, s3, h, stream=stream)
            ev[3].record(stream)
            moe.moe_expert_down_fp8(desc, T, h, counts, offsets, q2, s2, y_perm, stream=stream)
            ev[4].record(stream)
            moe.moe_combine(desc, y_perm, row_of, gate, y=y, stream=stream)
            ev[5].record(stream)
    else:
        def staged_step(ev):
            moe.moe_layer_forward_timed(desc, x, wg, w1, w3, w2, ev, y=y, topk_idx_out=idx, topk_gate_out=gate,
                                        counts_out=counts, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        layer_step()
    torch.cuda.synchronize()

    # Phase A: the reported value (mean over the synchronised window) and the
    # median of the per-step event intervals
    step_ev = events(args.steps + 1, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step_ev[s].record(stream)
        layer_step()
    step_ev[args.steps].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    ms_median = statistics.median(step_ev[s].elapsed_time(step_ev[s + 1]) for s in range(args.steps))

    # Phase B: per-stage durations from HIP events on the kernels' stream
    evs = [events(6, stream) for _ in range(args.steps)]
    torch.cuda.synchronize()
    tb0 = time.perf_counter()
    for s in range(args.steps):
        staged_step(evs[s])
    torch.cuda.synchronize()
    staged_ms = 1e3 * (time.perf_counter() - tb0) / args.steps
    stage_ms = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
                for i, name in enumerate(STAGES)}

    cnt = counts.cpu().tolist()
    touched = sum(1 for c in cnt if c > 0)
    TK = T * K
    esz = 2 if dt == torch.bfloat16 else 4
    wsz = 1 if fp8 else esz                     # bytes per expert weight
    ssz = 4 if fp8 else 0                       # bytes of scale per weight row
    # algorithmic work of the dominant kernel (gate/up + SwiGLU): per touched
    # expert 2*F*d weights (and their 2*F row scales), plus the gathered rows
    # read and h written
    gu_bytes = touched * 2 * F * (d * wsz + ssz) + TK * d * esz + TK * F * esz
    gu_flops = 4.0 * TK * d * F
    layer_bytes = touched * (3 * F * d * wsz + (2 * F + d) * ssz) + 2 * T * d * esz + d * n * 4
    layer_flops = 2.0 * TK * 3 * d * F + 2.0 * T * d * n
    gu_s = stage_ms["expert_gate_up"] / 1e3
    bound = "hbm" if (T * K) / max(1, touched) < 64 else "mfma"
    kern_name = ("gate_up_stream" if tile_m == 16 else "gate_up_tiled") if dt == torch.bfloat16 else "gate_up_f32"
    if fp8:
        kern_name = "gate_up_stream_fp8"
    if bound == "hbm":
        achieved = gu_bytes / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = gu_flops / gu_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = stored_traffic(kern_name, wl_name)
    roof["kernel"] = kern_name
    roof["kernel_ms"] = round(stage_ms["expert_gate_up"], 4)
    roof["algorithmic_per_launch"] = gu_bytes if bound == "hbm" else gu_flops

    layer_s = ms_per_step / 1e3
    out = {
        "metric": METRIC,
        "value": round(T / layer_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(ms_median, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl_name, "T": T, "d_model": d, "d_ffn": F, "n_experts": n,
                   "top_k": K, "tile_m": tile_m, "expert_weights": "fp8_e4m3" if fp8 else str(inp.dtype),
                   "expert_counts": cnt},
        "roofline": roof,
        "layer": {"hbm_GBs": round(layer_bytes / layer_s / 1e9, 1),
                  "hbm_frac": round(layer_bytes / layer_s / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_TFLOPs": round(layer_flops / layer_s / 1e12, 1),
                  "mfma_frac": round(layer_flops / layer_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                  "staged_ms_per_step": round(staged_ms, 4),
                  "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()}},
    }
    del x, wg, ws, y
    if not fp8:
        del w1, w3, w2
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_seconds > 0 and not fp8:  # the oracle's cost does not depend on the weight format
        out["cpu_baseline"] = cpu_baseline(inp, cpu_seconds, rows_cap=32 if wl <= 1 else 64)
    return out


def prefill_block(res: dict) -> dict:
    """The prefill workload's figures, as the "prefill" block of the default line."""
    keep = {k: res[k] for k in ("ms_per_step", "ms_per_step_median", "roofline")}
    keep["workload"] = res["config"]["workload"]
    keep["T"] = res["config"]["T"]
    keep["tokens_per_s"] = res["value"]
    keep["steps"], keep["warmup"] = res["steps"], res["warmup"]
    keep["layer_mfma_frac"] = res["layer"]["mfma_frac"]
    keep["layer_mfma_TFLOPs"] = res["layer"]["mfma_TFLOPs"]
    keep["stage_ms"] = res["layer"]["stage_ms"]
    keep["expert_counts"] = res["config"]["expert_counts"]
    if "cpu_baseline" in res:
        keep["cpu_baseline"] = res["cpu_baseline"]
    return keep


def bench_backward(args, spec):
    """Steps of moe_layer_backward between device synchronisations, then the
    same steps between HIP events on the launch stream."""
    import torch
    import moe_inputs as mi
    import sparse_moe_transformer_way_amd as moe

    inp = mi.make_workload(WORKLOADS["backward"], seed=args.seed)
    T, d, F, n, K = inp.T, inp.d, inp.F, inp.n, inp.K
    dev = torch.device("cuda")
    x, wg, w1, w3, w2 = (t.to(dev) for t in (inp.x, inp.wg, inp.w1, inp.w3, inp.w2))
    gen = torch.Generator(device=dev).manual_seed(args.seed + 1)
    dy = torch.randn((T, d), generator=gen, device=dev).to(torch.bfloat16)
    desc = moe.make_desc(d, F, n, K)
    dx = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    dwg = torch.empty((d, n), dtype=torch.float32, device=dev)
    dw1 = torch.empty((n, F, d), dtype=torch.float32, device=dev)
    dw3 = torch.empty((n, F, d), dtype=torch.float32, device=dev)
    dw2 = torch.empty((n, d, F), dtype=torch.float32, device=dev)
    ws = torch.empty(moe.moe_backward_workspace_size(desc, T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_layer_backward(desc, x, wg, w1, w3, w2, dy, dx, dwg, dw1, dw3, dw2, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    step_ev = events(args.steps + 1, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step_ev[s].record(stream)
        step()
    step_ev[args.steps].record(stream)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    ms_median = statistics.median(step_ev[s].elapsed_time(step_ev[s + 1]) for s in range(args.steps))
    ev = events(2, stream)
    ev[0].record(stream)
    for _ in range(args.steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ev_ms = ev[0].elapsed_time(ev[1]) / args.steps
    TK = T * K
    # five grouped products of 2 * TK * d * F flop each, two of them doubled (w1 and w3)
    flops = 16.0 * TK * d * F
    achieved = flops / (ev_ms / 1e3) / 1e12
    out = {
        "metric": "MoE-layer backward tokens/sec at 1 MI355X + % of MFMA roofline",
        "value": round(T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec["name"] + "_backward", "T": T, "d_model": d, "d_ffn": F, "n_experts": n,
                   "top_k": K, "weight_grads": "fp32"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "moe_layer_backward (all kernels of the pass)", "kernel_ms": round(ev_ms, 4),
                     "algorithmic_per_launch": flops},
    }
    print(json.dumps(out), flush=True)


def stack_cpu_baseline(layers, h0, seconds: float, n_rows: int = 256):
    """The oracle on a seeded sample of n_rows tokens followed block after block
    through the stack (tokens are independent with attention omitted), each
    layer's weights copied to the host when its turn comes, until `seconds` of
    oracle time have passed; stack tokens/s is scaled from the mean oracle time
    per block.  The host copies are not timed."""
    import numpy as np
    import oracle

    T = h0.shape[0]
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(T, size=min(n_rows, T), replace=False))
    hs = h0.float().cpu().numpy()[rows]
    spent = 0.0
    done = 0
    for wg, w1, w3, w2 in layers:
        wgn, w1n, w3n, w2n = (t.float().cpu().numpy() for t in (wg, w1, w3, w2))
        t0 = time.perf_counter()
        hs, _ = oracle.moe_block(hs, wgn, w1n, w3n, w2n)
        spent += time.perf_counter() - t0
        done += 1
        del w1n, w3n, w2n
        if spent >= seconds:
            break
    per_block = spent / done
    host = host_facts()
    return {"value": len(rows) / (per_block * len(layers)), "unit": "tokens/s", "cores": host["blas_threads"],
            "kind": "oracle",
            "sample": f"{len(rows)} of {T} tokens through the first {done} of {len(layers)} blocks (dense fp32, "
                      f"all experts), {spent:.1f} s of oracle time, scaled to {len(layers)} blocks",
            "host": host}


def bench_stack(args, spec):
    """Steps of the 32-block stack between device synchronisations, then the
    gate/up kernel of every layer between HIP events on the launch stream."""
    import torch
    import moe_inputs as mi
    import sparse_moe_transformer_way_amd as moe

    T, d, F, n, K, L = spec["T"], spec["d"], spec["F"], spec["n"], spec["K"], spec["layers"]
    dev = torch.device("cuda")
    layers = [mi.stack_layer_weights(l, d, F, n, seed=args.seed, device="cuda") for l in range(L)]
    h0 = mi.stack_input(T, d, seed=args.seed).to(dev)
    desc = moe.make_desc(d, F, n, K)
    tile_m = moe.moe_default_tile_m(desc, T)
    P = moe.moe_max_permuted_rows(desc, T, tile_m)
    h = torch.empty_like(h0)
    ws = torch.empty(moe.moe_block_workspace_size(desc, T), dtype=torch.uint8, device=dev)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    cnt = torch.empty((L, n), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step():
        # block 0 reads h0, the others update h in place
        for l, (wg, w1, w3, w2) in enumerate(layers):
            moe.moe_block_forward(desc, h0 if l == 0 else h, wg, w1, w3, w2, eps=1e-5, h_out=h,
                                  topk_idx_out=idx, counts_out=cnt[l], workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    step_ev = events(args.steps + 1, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step_ev[s].record(stream)
        step()
    step_ev[args.steps].record(stream)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    ms_median = statistics.median(step_ev[s].elapsed_time(step_ev[s + 1]) for s in range(args.steps))

    # the gate/up kernel of each layer, on that layer's routing of the stack's
    # last h states (normed input, router and permute run untimed first)
    x = torch.empty_like(h0)
    gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    counts = torch.empty(n, dtype=torch.int32, device=dev)
    offsets = torch.empty(n + 1, dtype=torch.int32, device=dev)
    row_src = torch.empty(P, dtype=torch.int32, device=dev)
    row_of = torch.empty((T, K), dtype=torch.int32, device=dev)
    hbuf = torch.empty((P, F), dtype=torch.bfloat16, device=dev)
    reps = max(1, min(args.steps, 5))
    ev = [events(2, stream) for _ in range(L * reps)]
    for r in range(reps):
        for l, (wg, w1, w3, w2) in enumerate(layers):
            moe.moe_rmsnorm(h, 1e-5, x_out=x, stream=stream)
            moe.moe_router_topk(desc, x, wg, idx, gate, stream=stream)
            moe.moe_permute(desc, idx, tile_m, counts, offsets, row_src, row_of, stream=stream)
            ev[r * L + l][0].record(stream)
            moe.moe_expert_gate_up(desc, T, tile_m, x, row_src, counts, offsets, w1, w3, hbuf, stream=stream)
            ev[r * L + l][1].record(stream)
    torch.cuda.synchronize()
    gu_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    TK = T * K
    gu_flops = 4.0 * TK * d * F
    achieved = gu_flops / (gu_ms / 1e3) / 1e12
    block_flops = 2.0 * TK * 3 * d * F + 2.0 * T * d * n
    out = {
        "metric": METRIC,
        "value": round(T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec["name"], "T": T, "layers": L, "d_model": d, "d_ffn": F, "n_experts": n,
                   "top_k": K, "tile_m": tile_m, "expert_counts_last_layer": cnt[L - 1].cpu().tolist()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic("gate_up_tiled", spec["name"]),
                     "kernel": "gate_up_tiled (mean over the layers)", "kernel_ms": round(gu_ms, 4),
                     "algorithmic_per_launch": gu_flops},
        "stack": {"layer_tokens_per_s": round(T * L / (ms / 1e3), 1), "ms_per_layer": round(ms / L, 4),
                  "mfma_frac": round(block_flops * L / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    del ws, hbuf, x
    torch.cuda.synchronize()
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = stack_cpu_baseline(layers, h0, max(args.cpu_seconds, 10.0))
    print(json.dumps(out), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch  # noqa: F401

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.vs_library:
        vs_library(args)
        return

    import moe_inputs as mi

    wl = WORKLOADS[args.workload]
    spec = mi.WORKLOADS[wl]
    if args.workload == "stack":
        bench_stack(args, spec)
        return
    if args.workload == "backward":
        bench_backward(args, spec)
        return
    out = run_layer(args, wl, args.workload == "decode_fp8", args.cpu_seconds)
    if args.workload == "decode" and not args.no_prefill:
        out["prefill"] = prefill_block(run_layer(args, WORKLOADS["prefill"], False, args.cpu_seconds))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
