#!/usr/bin/env python3
"""Benchmark: fused LoRA linear forward + backward on one MI355X.

One step = the whole hot path over one batch: the fused forward
(H = X W^T + s (X A^T) B^T, U saved) followed by the backward (dX, dA, dB),
for every linear of the workload (backward in reverse order).  Inputs are
resident in HBM before timing starts; several input sets are rotated so the
256 MB Infinity Cache cannot serve the operands of one step from the previous
one (cold operands, as in a training step where W was last touched a layer
stack ago).

Prints one JSON line.  Timing: W warm-up steps, then K timed steps between
device synchronisations, with HIP events recorded on the stream the library
launches on.  For a rank <= 16 layer the forward call is exactly one kernel
(the fused GEMM), so its event pair times that kernel alone: that is the
roofline figure.  The CPU baseline times the float64 oracle on a bounded
sample of the same workload on the host cores.

Extra modes (used to produce the committed counter summaries):
  --copy-calibration    run a plain device copy of known size (for scaling
                        the FETCH_SIZE / WRITE_SIZE counters)
  --traffic-from DIR    read rocprofv3 --pmc CSVs from DIR and write the
                        measured HBM traffic of the dominant kernel to
                        profiles/traffic_<workload>.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBPS = 8000.0             # MI355X HBM3E (published)
DEQUANT_SHAPE = (28672, 8192)      # the 4-bit layer's frozen weight, d_out x d_in
PEAK_HBM_GBS = 8000.0
METRIC = "fused LoRA linear fwd+bwd TFLOP/s and tokens/s; % bf16 MFMA peak (1 GPU)"
COPY_BYTES = 256 << 20             # calibration copy: 256 MiB read + 256 MiB written
# the sources of the kernel whose HBM traffic the counters measured (the fused GEMM)
KERNEL_SOURCES = ("lora_linear_layer_amd/csrc/lora_gemm.hpp", "lora_linear_layer_amd/csrc/common.hpp")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="attn_proj_4096")
    ap.add_argument("--input-sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dequant", action="store_true",
                    help="skip the stand-alone timings of the dequantisation and merge kernels")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of each step (captured once per input set)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time for the CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic-from", default=None)
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for pat in KERNEL_SOURCES:
        for p in sorted(glob.glob(os.path.join(ROOT, pat))):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def fwd_bytes(l) -> int:
    """HBM bytes a forward launch must move once: X and H in bf16, W in bf16
    or as 4-bit codes plus one fp16 absmax per 64 weights, A, B and the saved
    U (float32)."""
    w = l.N * l.K // 2 + 2 * (l.N * l.K // 64) if l.quant4 else 2 * l.N * l.K
    return 2 * l.M * l.K + w + 2 * l.M * l.N + 2 * l.r * (l.K + l.N) + 4 * l.M * l.r


def fwd_flops(l):
    return 2 * l.M * l.N * l.K + 2 * l.M * l.r * (l.K + l.N)


def bwd_flops(l):
    return 2 * l.M * l.N * l.K + 4 * l.M * l.r * (l.K + l.N)


def cpu_baseline(wl, min_seconds):
    """The float64 oracle's forward + backward on the first linear of the
    workload (all of its tokens), repeated until min_seconds have passed."""
    import numpy as np  # noqa: F401
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max(int(p.get("num_threads", 1)) for p in info) if info else 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    sh = wl.linears[0]
    inp = workloads.make_qlora_inputs(sh) if sh.quant4 else workloads.make_linear_inputs(sh)
    if sh.quant4:
        W = oracle.dequant4(inp["codes"], inp["absmax"], oracle.codebook4())
    else:
        W = inp["W"]
    s = sh.scale
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(inp["X"], W, inp["A"], inp["B"], s)
        oracle.backward(inp["dY"], inp["X"], W, inp["A"], inp["B"], s)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    flops = runs * sh.flops()
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2), "tokens_per_s": round(runs * sh.M / dt, 1),
            "sample": f"{sh.name}: all {sh.M} tokens, K={sh.K}, N={sh.N}, r={sh.r}, float64 numpy forward+backward, "
                      f"{runs} run(s) ({sh.flops() / 1e9:.1f} GFLOP each)"
                      + ("; 4-bit weights dequantised once beforehand, not timed" if sh.quant4 else "")}


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def load_traffic(workload):
    p = traffic_path(workload)
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None          # the kernels changed since the counters were taken
    return t


def write_traffic(args):
    """Mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the dominant kernel and
    of the calibration copy, from rocprofv3 --pmc counter_collection CSVs."""
    def mean_counter(prefix, counter, pred):
        vals = []
        for f in glob.glob(os.path.join(args.traffic_from, prefix + "*counter_collection.csv")):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] == counter and pred(row["Kernel_Name"]):
                    vals.append(float(row["Counter_Value"]))
        return sum(vals) / len(vals) if vals else None

    # bench_* files: the forward GEMM (first template argument false); copy_* files: the neg kernel
    is_gemm = lambda k: "lora_gemm" in k and k.split("<", 1)[-1].split(",")[0].strip() == "false"
    is_copy = lambda k: "neg_kernel" in k
    fetch_k, write_k = mean_counter("bench_", "FETCH_SIZE", is_gemm), mean_counter("bench_", "WRITE_SIZE", is_gemm)
    cfetch_k, cwrite_k = mean_counter("copy_", "FETCH_SIZE", is_copy), mean_counter("copy_", "WRITE_SIZE", is_copy)
    if None in (fetch_k, write_k, cfetch_k, cwrite_k):
        raise SystemExit("missing counters: need FETCH_SIZE and WRITE_SIZE runs of both the bench and the copy")
    f_fac = cfetch_k * 1024 / COPY_BYTES
    w_fac = cwrite_k * 1024 / COPY_BYTES
    out = {"workload": args.workload, "kernel": "lora_gemm forward", "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_dispatch": fetch_k, "write_kib_per_dispatch": write_k,
           "copy_kib_fetch": cfetch_k, "copy_kib_write": cwrite_k, "copy_bytes": COPY_BYTES,
           "copy_fetch_factor": round(f_fac, 4), "copy_write_factor": round(w_fac, 4),
           "hbm_read_bytes_per_dispatch": round(fetch_k * 1024 / f_fac),
           "hbm_write_bytes_per_dispatch": round(write_k * 1024 / w_fac),
           "hbm_bytes_per_dispatch": round(fetch_k * 1024 / f_fac + write_k * 1024 / w_fac)}
    os.makedirs(os.path.dirname(traffic_path(args.workload)), exist_ok=True)
    json.dump(out, open(traffic_path(args.workload), "w"), indent=1)
    print(json.dumps(out))


def dequant_rate(lla, workloads, torch, dev, stream, reps=20):
    """The stand-alone 4-bit dequantisation (lora_dequant4, bf16 output) on the
    4-bit layer's weight shape: HIP events on the library's stream around each
    launch; bytes = codes (0.5 B) + fp16 absmax (2 B per 64) + bf16 out (2 B)
    per weight, each moved once."""
    N, K = DEQUANT_SHAPE
    g = torch.Generator(device=dev)
    g.manual_seed(4004)
    codes = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=g)
    absmax = (torch.rand((N, K // 64), device=dev, generator=g) * 0.08 + 0.01).to(torch.float16).view(torch.int16)
    cb = torch.from_numpy(workloads.codebook4_f32()).to(dev)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    run = lambda: lla.lora_dequant4(codes, absmax, cb, N, K, lla.LORA_DTYPE_BF16, out, stream=stream)
    for _ in range(3):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3
    nbytes = N * K // 2 + 2 * (N * K // 64) + 2 * N * K
    gbps = nbytes / (us * 1e-6) / 1e9
    del codes, absmax, out
    return {"kernel": "dequant4_kernel (lora_dequant4, bf16 out)", "shape": [N, K], "bound": "hbm",
            "bytes_per_launch": nbytes, "avg_launch_us": round(us, 2), "achieved": round(gbps, 1),
            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}


def merge_rate(lla, torch, dev, stream, l, reps=20):
    """lora_merge (W_out = W + s B A, bf16, out of place) on the weight shape of
    linear l: HIP events on the library's stream around each launch; bytes =
    W read and W_out written once (2 + 2 bytes per weight) plus A and B."""
    g = torch.Generator(device=dev)
    g.manual_seed(5005)
    W = (torch.randn((l.N, l.K), device=dev, generator=g) * 0.02).to(torch.bfloat16)
    A = (torch.randn((l.r, l.K), device=dev, generator=g) * l.K ** -0.5).to(torch.bfloat16)
    B = (torch.randn((l.N, l.r), device=dev, generator=g) * 0.02).to(torch.bfloat16)
    out = torch.empty_like(W)
    desc = lla.Desc(1, l.K, l.N, l.r, l.alpha)
    run = lambda: lla.lora_merge(desc, W, A, B, out, 1, stream=stream)
    for _ in range(3):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3
    nbytes = 4 * l.N * l.K + 2 * l.r * (l.K + l.N)
    gbps = nbytes / (us * 1e-6) / 1e9
    del W, A, B, out
    return {"kernel": "lora_merge_kernel (lora_merge, bf16)", "shape": [l.N, l.K, l.r], "bound": "hbm",
            "bytes_per_launch": nbytes, "avg_launch_us": round(us, 2), "achieved": round(gbps, 1),
            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}


def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)        # one elementwise kernel: reads and writes COPY_BYTES
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py runs on exactly one GPU; --gpus must be 1 "
                                   "(data-parallel sharding across GPUs is not built)"}))
        sys.exit(2)
    if args.traffic_from:
        write_traffic(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return

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
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # the library launches on the stream torch reports as current (the capture
    # stream while a graph is being recorded)
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
    mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev_f = [[mk() for _ in range(n_lin)] for _ in range(args.steps)]
    ev_b = [[mk() for _ in range(n_lin)] for _ in range(args.steps)]

    def step(i, timed):
        layer = sets[i % len(sets)]
        for li, d in enumerate(layer):
            if timed:
                ev_f[i][li][0].record(stream)
            fwd(d)
            if timed:
                ev_f[i][li][1].record(stream)
        for li in reversed(range(n_lin)):
            if timed:
                ev_b[i][li][0].record(stream)
            bwd(layer[li])
            if timed:
                ev_b[i][li][1].record(stream)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    run = lambda i: step(i, False)
    if args.graph:
        graphs = []
        for si in range(len(sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(si, False)
            graphs.append(g)
        torch.cuda.synchronize()
        run = lambda i: graphs[i % len(graphs)].replay()
        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()
    # the timed region holds only the steps themselves (no per-call events)
    t_start, t_end = mk()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        run(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    # per-call durations (per-linear table, roofline) from a second pass of the
    # same steps with HIP events around every library call
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()

    flops = wl.flops()
    tflops = flops / (ms_step * 1e-3) / 1e12
    tokens_s = wl.tokens / (ms_step * 1e-3)

    def mean_ms(ev, li):
        return sum(ev[i][li][0].elapsed_time(ev[i][li][1]) for i in range(args.steps)) / args.steps

    per_linear = []
    for li, l in enumerate(wl.linears):
        f_ms, b_ms = mean_ms(ev_f, li), mean_ms(ev_b, li)
        per_linear.append({"name": l.name, "fwd_us": round(f_ms * 1e3, 2), "bwd_us": round(b_ms * 1e3, 2),
                           "fwd_tflops": round(fwd_flops(l) / (f_ms * 1e-3) / 1e12, 1),
                           "bwd_tflops": round(bwd_flops(l) / (b_ms * 1e-3) / 1e12, 1)})

    # dominant kernel: the fused forward GEMM of the largest linear
    big = max(range(n_lin), key=lambda i: fwd_flops(wl.linears[i]))
    lb = wl.linears[big]
    fwd_ms = mean_ms(ev_f, big)
    ach = fwd_flops(lb) / (fwd_ms * 1e-3) / 1e12
    tr = load_traffic(wl.name)
    roofline = {"kernel": f"lora_gemm forward ({lb.name})" + ("" if lb.r <= 16 else " + skinny U pass"),
                "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": tr["hbm_bytes_per_dispatch"] if tr else None,
                "avg_launch_us": round(fwd_ms * 1e3, 2), "flops_per_launch": fwd_flops(lb),
                "algorithmic_bytes_per_launch": fwd_bytes(lb)}

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "launch": "hip_graph_replay" if args.graph else "eager",
        "data": "synthetic (seeded on-device normal draws; no dataset or checkpoint)",
        "config": {"workload": wl.name, "linears": [[l.name, l.M, l.K, l.N, l.r, l.alpha] for l in wl.linears],
                   "input_sets": args.input_sets, "description": wl.description},
        "tokens_per_s": round(tokens_s, 1), "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "algorithmic_gflop_per_step": round(flops / 1e9, 3), "wall_s_timed": round(wall, 3),
        "per_linear": per_linear,
        "roofline": roofline,
    }
    if not args.no_dequant:
        out["hbm_kernels"] = [dequant_rate(lla, workloads, torch, dev, stream),
                              merge_rate(lla, torch, dev, stream, lb)]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
