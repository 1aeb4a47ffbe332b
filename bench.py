#!/usr/bin/env python3
"""Benchmark: fused LoRA linear forward + backward on one MI355X.

One step = the whole hot path over one batch: the fused forward
(H = X W^T + s (X A^T) B^T, U saved) followed by the backward (dX, dA, dB),
for every linear of the workload (backward in reverse order).  Inputs are
resident in HBM before timing starts; several input sets are rotated so the
256 MB Infinity Cache cannot hold the whole working set between steps.

Prints one JSON line (rank 0).  Timing: W warm-up steps, then K timed steps
between device synchronisations, with HIP events on the stream the kernels are
launched on.  The forward call of a rank <= 64 layer is exactly one kernel
(the fused GEMM), so its event pair times that kernel alone: that is the
roofline figure.  The CPU baseline times the float64 oracle on a bounded
sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0
METRIC = "fused LoRA linear fwd+bwd TFLOP/s and tokens/s; % bf16 MFMA peak (1 GPU)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="attn_proj_4096")
    ap.add_argument("--input-sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=512)
    return ap.parse_args()


def fwd_flops(l):
    return 2 * l.M * l.N * l.K + 2 * l.M * l.r * (l.K + l.N)


def cpu_baseline(wl, rows):
    """Oracle (numpy float64) forward + backward on the first `rows` tokens of the
    workload's first linear; reported in TFLOP/s of algorithmic work."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max(int(p.get("num_threads", 1)) for p in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    sh = wl.linears[0]
    inp = workloads.make_linear_inputs(sh)
    X, dY = inp["X"][:rows], inp["dY"][:rows]
    s = sh.scale
    t0 = time.perf_counter()
    if sh.quant4:
        W = oracle.dequant4(*workloads.quantize4(inp["W"]), oracle.codebook4())
    else:
        W = inp["W"]
    t_deq = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.forward(X, W, inp["A"], inp["B"], s)
    oracle.backward(dY, X, W, inp["A"], inp["B"], s)
    dt = time.perf_counter() - t0
    sample_flops = 4 * rows * sh.N * sh.K + 6 * rows * sh.r * (sh.K + sh.N)
    return {"value": sample_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{sh.name}: first {rows} of {sh.M} tokens, K={sh.K}, N={sh.N}, r={sh.r}, float64 numpy "
                      f"forward+backward ({sample_flops / 1e9:.1f} GFLOP)"
                      + (f"; 4-bit dequant of W took {t_deq:.1f}s, not counted" if sh.quant4 else "")}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1 "
                                   "(data-parallel sharding is described in DESIGN.md, not built)"}))
        sys.exit(2)

    import torch
    import lora_linear_layer_amd as lla
    import workloads

    wl = workloads.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---------------------------------------------------------------- inputs
    sets = []
    for si in range(args.input_sets):
        layer = []
        shared_x = {}
        for li, sh in enumerate(wl.linears):
            d = workloads.device_inputs_torch(sh, dev, torch.bfloat16, seed=sh.seed * 100 + si)
            if sh.quant4:
                d.update(workloads.quantize4_torch(d.pop("W").float()))
            # q/k/v share one input, gate/up share one input (decoder layer)
            key = sh.name.split("_")[-1]
            group = {"q": "qkv", "k": "qkv", "v": "qkv", "gate": "gu", "up": "gu"}.get(key)
            if group:
                if group in shared_x:
                    d["X"] = shared_x[group]
                else:
                    shared_x[group] = d["X"]
            desc = lla.Desc(sh.M, sh.K, sh.N, sh.r, sh.alpha)
            d["desc"] = desc
            d["H"] = torch.empty((sh.M, sh.N), dtype=torch.bfloat16, device=dev)
            d["U"] = torch.empty((sh.M, sh.r), dtype=torch.float32, device=dev)
            d["dX"] = torch.empty((sh.M, sh.K), dtype=torch.bfloat16, device=dev)
            d["dA"] = torch.empty((sh.r, sh.K), dtype=torch.bfloat16, device=dev)
            d["dB"] = torch.empty((sh.N, sh.r), dtype=torch.bfloat16, device=dev)
            layer.append(d)
        sets.append(layer)
    ws_bytes = max(lla.lora_linear_workspace_size(d["desc"]) for d in sets[0])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def fwd(d):
        if "codes" in d:
            lla.lora_qlinear_fwd(d["desc"], d["X"], d["codes"], d["absmax"], d["codebook"], d["A"], d["B"],
                                 d["H"], d["U"], ws=ws, ws_bytes=ws_bytes)
        else:
            lla.lora_linear_fwd(d["desc"], d["X"], d["W"], d["A"], d["B"], d["H"], d["U"], ws=ws,
                                ws_bytes=ws_bytes)

    def bwd(d):
        if "codes" in d:
            lla.lora_qlinear_bwd(d["desc"], d["dY"], d["X"], d["codes"], d["absmax"], d["codebook"], d["A"],
                                 d["B"], d["U"], d["dX"], d["dA"], d["dB"], ws=ws, ws_bytes=ws_bytes)
        else:
            lla.lora_linear_bwd(d["desc"], d["dY"], d["X"], d["W"], d["A"], d["B"], d["U"], d["dX"], d["dA"],
                                d["dB"], ws=ws, ws_bytes=ws_bytes)

    n_lin = len(wl.linears)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_lin)]
          for _ in range(args.steps)]

    def step(i, timed):
        layer = sets[i % len(sets)]
        for li, d in enumerate(layer):
            if timed:
                ev[i][li][0].record(stream)
            fwd(d)
            if timed:
                ev[i][li][1].record(stream)
        for d in reversed(layer):
            bwd(d)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(i, True)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps

    flops = wl.flops()
    tflops = flops / (ms_step * 1e-3) / 1e12
    tokens_s = wl.tokens / (ms_step * 1e-3)

    # dominant kernel: the fused forward GEMM of the largest linear (one launch per call)
    big = max(range(n_lin), key=lambda i: fwd_flops(wl.linears[i]))
    fwd_ms = sum(ev[i][big][0].elapsed_time(ev[i][big][1]) for i in range(args.steps)) / args.steps
    lb = wl.linears[big]
    ach = fwd_flops(lb) / (fwd_ms * 1e-3) / 1e12
    roofline = {"kernel": f"fused_lora_gemm forward ({lb.name})", "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": None, "avg_launch_us": round(fwd_ms * 1e3, 2),
                "flops_per_launch": fwd_flops(lb)}

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded on-device normal draws; no dataset or checkpoint)",
        "config": {"workload": wl.name, "linears": [[l.name, l.M, l.K, l.N, l.r, l.alpha] for l in wl.linears],
                   "input_sets": args.input_sets, "description": wl.description},
        "tokens_per_s": round(tokens_s, 1), "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "algorithmic_gflop_per_step": round(flops / 1e9, 3),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, min(args.cpu_sample_rows, wl.linears[0].M))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
