#!/usr/bin/env python3
"""Benchmark: fused LoRA linear forward + backward on one MI355X.

One step = the whole hot path over one batch: the fused forward
(H = X W^T + s (X A^T) B^T, U saved) followed by the backward (dX, dA, dB),
for every linear of the workload (forwards in order, backwards in reverse,
one shared workspace).  Inputs are resident in HBM before timing starts;
several input sets are rotated so the 256 MB Infinity Cache cannot serve the
operands of one step from the previous one (cold operands, as in a training
step where W was last touched a layer stack ago).

Before the counted warm-up, the steps run for --device-warmup-s seconds of
wall time (default 0.3 s; reported as `device_warmup`): the MI355X raises its
clocks only under sustained load, so a few warm-up steps after idle measure
the ramp (0.285 ms per step at the 4096 projection after 5 steps, 0.245 ms
after 300, same binary and call), while a training loop runs in the steady
state.  The timed region is unaffected: exactly K full steps.

Prints one JSON line.  Timing passes, both on the stream the library launches on:
  1. the timed region: W warm-up steps, then K steps between two HIP events,
     device-synchronised on both sides, nothing else inside (`value`);
  2. the same K steps again with the library's kernel timer set: HIP events
     attached to every kernel's dispatch (hipExtLaunchKernel) record its start
     and end without adding commands between the kernels, so the kernels run
     back to back as in the timed region.  They give each kernel's mean
     duration (the roofline entries of the GEMMs; the dominant kernel,
     `roofline`, is the GEMM with the largest measured time per step) and the
     spread of the step time, first kernel start to last kernel end
     (p10 / p50 / p90).
The CPU baseline times the float64 oracle on a bounded sample of the same
workload on the host cores.

Extra modes (used to produce the committed counter summaries):
  --copy-calibration    run a plain device copy of known size (for scaling
                        the FETCH_SIZE / WRITE_SIZE counters)
  --traffic-from DIR    read rocprofv3 --pmc CSVs from DIR and write the
                        measured HBM traffic of both GEMMs to
                        profiles/traffic_<workload>.json
  --grouped             run the linears that read the same input (q/k/v,
                        gate/up) as one grouped call each (lora_group_fwd /
                        lora_group_bwd: one pass over X for all their U, one
                        GEMM over the stacked weights, the shared input's
                        gradient summed over them)
  --w-layout {wt,w}     the frozen weight the backward reads: wt (default)
                        W^T [K, N], transposed once before timing and kept
                        beside W (LORA_FLAG_W_TRANSPOSED: the input-gradient
                        GEMM then reads it in the forward's layout); w: W
                        itself, gathered with transposing LDS reads.  4-bit
                        weights always use their codes.
  --norm                the linears that read a normalised input (the
                        projection of attn_proj_4096; q/k/v and gate/up)
                        run with the RMSNorm in front (lora_norm_linear_* /
                        lora_norm_group_*: the layer reads the raw X, W is
                        folded with the norm weight once before timing, dX
                        is the gradient through the norm).  The norm's own
                        O(M K) arithmetic is not counted in the FLOPs, its
                        kernels' time is in the step.
"""
from __future__ import annotations

import argparse
import ctypes
import csv
import dataclasses
import glob
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBPS = 8000.0             # MI355X HBM3E (published)
DEQUANT_SHAPE = (28672, 8192)      # the 4-bit layer's frozen weight, d_out x d_in
METRIC = "fused LoRA linear fwd+bwd TFLOP/s and tokens/s; % bf16 MFMA peak (1 GPU)"
COPY_BYTES = 256 << 20             # calibration copy: 256 MiB read + 256 MiB written
# the sources of the kernels whose HBM traffic the counters measured (the fused GEMMs)
KERNEL_SOURCES = ("lora_linear_layer_amd/csrc/lora_gemm.hpp", "lora_linear_layer_amd/csrc/common.hpp",
                  "lora_linear_layer_amd/csrc/ranges.hpp")
GEMM_FWD, GEMM_DX = "lora_gemm forward", "lora_gemm dX"
# linears that read the same input (decoder layer): q/k/v share X, gate/up share X
SHARED_INPUT = {"q": "qkv", "k": "qkv", "v": "qkv", "gate": "gu", "up": "gu"}
# linears whose input is an RMSNorm output: the attention projections behind
# the attention norm and gate/up behind the MLP norm (o and down read the
# attention and SwiGLU outputs); the single 4096 projection stands for q
NORM_EPS = 1e-6
NORM_KERNELS = ("norm_prep", "norm_fold", "norm_dx")


def behind_norm(name: str) -> bool:
    return name == "attn_proj_4096" or name.split("_")[-1] in SHARED_INPUT


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="attn_proj_4096")
    ap.add_argument("--input-sets", type=int, default=4)
    ap.add_argument("--device-warmup-s", type=float, default=0.3,
                    help="seconds of steps before the counted warm-up, to reach the steady clock (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dequant", action="store_true",
                    help="skip the stand-alone timings of the dequantisation and merge kernels")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of each step (captured once per input set)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time for the CPU baseline")
    ap.add_argument("--tune", action="store_true",
                    help="probe and cache the launch parameters of every single-linear call before timing "
                         "(lora_tune_linear; the probing is outside the timed region)")
    ap.add_argument("--grouped", action="store_true",
                    help="linears sharing an input run as one grouped call (q/k/v, gate/up)")
    ap.add_argument("--w-layout", choices=("wt", "w"), default="wt",
                    help="backward weight operand: W^T made once before timing (default), or W")
    ap.add_argument("--norm", action="store_true",
                    help="RMSNorm in front of the linears that read a normalised input")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor GEMM (torch.matmul) on the first linear's X W^T, for reference")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic-from", default=None)
    return ap.parse_args(argv)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for pat in KERNEL_SOURCES:
        for p in sorted(glob.glob(os.path.join(ROOT, pat))):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ counts
def w_bytes(l) -> int:
    """The frozen weight once: bf16, or 4-bit codes plus one fp16 absmax per 64 weights."""
    return l.N * l.K // 2 + 2 * (l.N * l.K // 64) if l.quant4 else 2 * l.N * l.K


def fwd_bytes(l) -> int:
    """HBM bytes a forward launch must move once: X and H in bf16, W, A, B and
    the saved U (float32)."""
    return 2 * l.M * l.K + w_bytes(l) + 2 * l.M * l.N + 2 * l.r * (l.K + l.N) + 4 * l.M * l.r


def fwd_flops(l):
    return 2 * l.M * l.N * l.K + 2 * l.M * l.r * (l.K + l.N)


def bwd_flops(l):
    return 2 * l.M * l.N * l.K + 4 * l.M * l.r * (l.K + l.N)


def in_tile(l, split: bool, dx: bool) -> bool:
    """Whether the GEMM forms its rank-r product itself (the library's rule:
    a plain layer, r <= 16, 16-bit W, whole tiles; the input gradient also
    needs r % 8 == 0)."""
    G = getattr(l, "G", 1)
    return G == 1 and l.r <= 16 and not l.quant4 and not split and (not dx or l.r % 8 == 0)


def gemm_flops(l, label: str) -> int:
    """Algorithmic FLOPs of one launch of a fused GEMM: the dense product,
    the rank-r term of the epilogue (a group: each output column's member
    rank r forward, the stacked rank G r in the input gradient) and, when
    formed in the tile, the rank-r product U = X A^T or V = dY B."""
    dx = label.startswith(GEMM_DX)
    G = getattr(l, "G", 1)
    P, Q, C = (l.M, l.K, l.N) if dx else (l.M, l.N, l.K)
    f = 2 * P * Q * C + 2 * P * Q * (G * l.r if dx else l.r)
    if in_tile(l, "(split)" in label, dx):
        f += 2 * P * l.r * C
    return f


def gemm_bytes(l, label: str) -> int:
    """Algorithmic HBM bytes of one launch of a fused GEMM, each operand once.
    Forward: X, W, A, B, H, and U (written, or read when precomputed).
    Input gradient: dY, W, A, B, dX, and U read; in the in-tile form also the
    four bf16 rank planes (V^T and U^T, hi and lo, r x M each) it writes,
    otherwise V read."""
    G = getattr(l, "G", 1)
    M, K, N, r, R = l.M, l.K, l.N, l.r, getattr(l, "G", 1) * l.r
    if not label.startswith(GEMM_DX):
        return 2 * M * K + w_bytes(l) + 2 * M * N + 2 * R * K + 2 * N * r + 4 * M * R
    b = 2 * M * N + w_bytes(l) + 2 * M * K + 2 * R * K + 2 * N * r + 4 * M * R
    if in_tile(l, "(split)" in label, True):
        b += 4 * 2 * r * (-(-M // 128) * 128)
    else:
        b += 4 * M * R
    return b


@dataclasses.dataclass(frozen=True)
class Unit:
    """What one library call of a step covers: a single linear (G = 1), or
    G linears that share their input, run as one group (N = their total)."""
    name: str
    M: int
    K: int
    N: int
    r: int
    alpha: float
    G: int = 1
    quant4: bool = False
    members: tuple = ()


def step_units(wl, grouped: bool):
    """The workload's linears as the calls of one step: consecutive linears of
    one shared-input set form a group when grouped is set."""
    units, i = [], 0
    lins = wl.linears
    while i < len(lins):
        l = lins[i]
        grp = SHARED_INPUT.get(l.name.split("_")[-1])
        j = i + 1
        if grouped and grp:
            while j < len(lins) and SHARED_INPUT.get(lins[j].name.split("_")[-1]) == grp:
                j += 1
        mem = lins[i:j]
        if len(mem) == 1:
            units.append(Unit(l.name, l.M, l.K, l.N, l.r, l.alpha, 1, l.quant4, (i,)))
        else:
            units.append(Unit("+".join(m.name for m in mem), l.M, l.K, sum(m.N for m in mem), l.r, l.alpha,
                              len(mem), False, tuple(range(i, j))))
        i = j
    return units


# ------------------------------------------------------------------ oracle baseline
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


# ------------------------------------------------------------------ traffic counters
def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def load_traffic(workload, w_layout="wt"):
    """Measured HBM bytes per dispatch of each GEMM, {label: bytes}, or None
    when no counters were taken for the current kernel sources and the same
    backward weight layout."""
    p = traffic_path(workload)
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None          # the kernels changed since the counters were taken
    if t.get("w_layout", "w") != w_layout:
        return None          # counters of the other input-gradient GEMM
    return {k: v["hbm_bytes_per_dispatch"] for k, v in t.get("kernels", {}).items()}


def write_traffic(args):
    """Mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of both GEMMs and of the
    calibration copy, from rocprofv3 --pmc counter_collection CSVs."""
    def mean_counter(prefix, counter, pred):
        vals = []
        for f in glob.glob(os.path.join(args.traffic_from, prefix + "*counter_collection.csv")):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] == counter and pred(row["Kernel_Name"]):
                    vals.append(float(row["Counter_Value"]))
        return sum(vals) / len(vals) if vals else None

    # bench_* files: the GEMMs (first template argument false: forward, true: input
    # gradient); copy_* files: the neg kernel
    def is_gemm(trans):
        def pred(k):
            if "lora_gemm<" not in k:
                return False
            targs = [a.strip() for a in k.split("lora_gemm<", 1)[1].split(">", 1)[0].split(",")]
            return targs[0] == trans
        return pred
    is_copy = lambda k: "neg_kernel" in k
    cfetch_k, cwrite_k = mean_counter("copy_", "FETCH_SIZE", is_copy), mean_counter("copy_", "WRITE_SIZE", is_copy)
    if None in (cfetch_k, cwrite_k):
        raise SystemExit("missing counters: need FETCH_SIZE and WRITE_SIZE runs of the copy")
    f_fac = cfetch_k * 1024 / COPY_BYTES
    w_fac = cwrite_k * 1024 / COPY_BYTES
    kernels = {}
    for label, trans in ((GEMM_FWD, "false"), (GEMM_DX, "true")):
        fetch_k = mean_counter("bench_", "FETCH_SIZE", is_gemm(trans))
        write_k = mean_counter("bench_", "WRITE_SIZE", is_gemm(trans))
        if None in (fetch_k, write_k):
            continue
        kernels[label] = {"fetch_kib_per_dispatch": fetch_k, "write_kib_per_dispatch": write_k,
                          "hbm_read_bytes_per_dispatch": round(fetch_k * 1024 / f_fac),
                          "hbm_write_bytes_per_dispatch": round(write_k * 1024 / w_fac),
                          "hbm_bytes_per_dispatch": round(fetch_k * 1024 / f_fac + write_k * 1024 / w_fac)}
    if not kernels:
        raise SystemExit("missing counters: need FETCH_SIZE and WRITE_SIZE runs of the bench")
    out = {"workload": args.workload, "kernel_source_hash": kernel_source_hash(), "w_layout": args.w_layout,
           "copy_kib_fetch": cfetch_k, "copy_kib_write": cwrite_k, "copy_bytes": COPY_BYTES,
           "copy_fetch_factor": round(f_fac, 4), "copy_write_factor": round(w_fac, 4), "kernels": kernels}
    os.makedirs(os.path.dirname(traffic_path(args.workload)), exist_ok=True)
    json.dump(out, open(traffic_path(args.workload), "w"), indent=1)
    print(json.dumps(out))


# ------------------------------------------------------------------ the step
def share_inputs(wl, layer):
    """Linears that read the same activations get the same X tensor: the first
    member of each group (q of q/k/v, gate of gate/up) provides it."""
    first = {}
    for sh, d in zip(wl.linears, layer):
        group = SHARED_INPUT.get(sh.name.split("_")[-1])
        if group is None:
            continue
        if group in first:
            d["X"] = first[group]
        else:
            first[group] = d["X"]
    return layer


def add_outputs(lla, torch, wl, layer, dev):
    """Descriptor and output buffers (H, U, dX, dA, dB) for each linear."""
    for sh, d in zip(wl.linears, layer):
        d["desc"] = lla.Desc(sh.M, sh.K, sh.N, sh.r, sh.alpha)
        d["H"] = torch.empty((sh.M, sh.N), dtype=torch.bfloat16, device=dev)
        d["U"] = torch.empty((sh.M, sh.r), dtype=torch.float32, device=dev)
        d["dX"] = torch.empty((sh.M, sh.K), dtype=torch.bfloat16, device=dev)
        d["dA"] = torch.empty((sh.r, sh.K), dtype=torch.bfloat16, device=dev)
        d["dB"] = torch.empty((sh.N, sh.r), dtype=torch.bfloat16, device=dev)
    return layer


def add_norm(lla, torch, wl, layer, dev, seed):
    """RMSNorm in front of the linears behind_norm selects: one norm weight g
    per shared input (the same tensor for q/k/v, and for gate/up), W folded
    with it in place (once, before timing), a saved 1/rms buffer per linear."""
    import workloads
    gs = {}
    for sh, d in zip(wl.linears, layer):
        if not behind_norm(sh.name):
            continue
        key = SHARED_INPUT.get(sh.name.split("_")[-1], sh.name)
        if key not in gs:
            gs[key] = workloads.norm_weight_torch(sh.K, dev, torch.bfloat16, seed + len(gs))
        d["g"] = gs[key]
        lla.lora_fold_norm_weight(d["W"], d["g"], d["W"])
        d["inv"] = torch.empty((sh.M,), dtype=torch.float32, device=dev)
    return layer


def add_wt(lla, torch, wl, layer):
    """W^T of every 16-bit frozen weight (made once, before any timing; after
    add_norm, so that it is the folded weight's transpose), and the flag that
    makes the backward read it."""
    for sh, d in zip(wl.linears, layer):
        if "W" not in d:
            continue
        d["Wt"] = torch.empty((sh.K, sh.N), dtype=d["W"].dtype, device=d["W"].device)
        lla.lora_transpose_weight(d["W"], d["Wt"])
        d["desc"] = dataclasses.replace(d["desc"], flags=d["desc"].flags | lla.LORA_FLAG_W_TRANSPOSED)
    return layer


def group_layer(lla, torch, wl, layer, units, dev):
    """The per-linear inputs of one step regrouped as units: a group's W, A, B
    and dY stacked (copies made once, before any timing), its outputs H
    [M][sum N], U [M][G r], dX [M][K] (the shared input's gradient, summed
    over the members), dA [G r][K], dB [sum N][r]."""
    out = []
    for u in units:
        if u.G == 1:
            out.append(layer[u.members[0]])
            continue
        ds = [layer[i] for i in u.members]
        g = {"gdesc": lla.GroupDesc(u.M, u.K, tuple(wl.linears[i].N for i in u.members), u.r, u.alpha),
             "X": ds[0]["X"],
             "W": torch.cat([d["W"] for d in ds]).contiguous(), "A": torch.cat([d["A"] for d in ds]).contiguous(),
             "B": torch.cat([d["B"] for d in ds]).contiguous(),
             "dY": torch.cat([d["dY"] for d in ds], dim=1).contiguous()}
        if "g" in ds[0]:
            g["g"] = ds[0]["g"]
            g["inv"] = ds[0]["inv"]
        if "Wt" in ds[0]:                    # the stacked weight's transpose [K][sum N]
            g["Wt"] = torch.cat([d["Wt"] for d in ds], dim=1).contiguous()
            g["gdesc"] = dataclasses.replace(g["gdesc"], flags=g["gdesc"].flags | lla.LORA_FLAG_W_TRANSPOSED)
        R = u.G * u.r
        g["H"] = torch.empty((u.M, u.N), dtype=torch.bfloat16, device=dev)
        g["U"] = torch.empty((u.M, R), dtype=torch.float32, device=dev)
        g["dX"] = torch.empty((u.M, u.K), dtype=torch.bfloat16, device=dev)
        g["dA"] = torch.empty((R, u.K), dtype=torch.bfloat16, device=dev)
        g["dB"] = torch.empty((u.N, u.r), dtype=torch.bfloat16, device=dev)
        out.append(g)
    return out


class Stepper:
    """Runs one step of a workload through the C ABI: every linear's fused
    forward in order, then every backward in reverse order, all on torch's
    current stream, with one workspace sized for the largest descriptor
    shared by all calls (and by all input sets)."""

    def __init__(self, lla, torch, layers, dev):
        self.lla = lla
        self.ws_bytes = max(self.ws_size(d) for layer in layers for d in layer)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.current = None          # index of the linear being run (for the per-kernel timing pass)

    def ws_size(self, d):
        lla = self.lla
        if "gdesc" in d:
            return (lla.lora_norm_group_workspace_size if "g" in d else lla.lora_group_workspace_size)(d["gdesc"])
        return (lla.lora_norm_linear_workspace_size if "g" in d else lla.lora_linear_workspace_size)(d["desc"])

    def fwd(self, d):
        lla = self.lla
        if "g" in d:
            f = lla.lora_norm_group_fwd if "gdesc" in d else lla.lora_norm_linear_fwd
            f(d.get("gdesc") or d["desc"], NORM_EPS, d["X"], d["g"], d["W"], d["A"], d["B"], d["H"], d["U"],
              d["inv"], ws=self.ws, ws_bytes=self.ws_bytes)
        elif "gdesc" in d:
            lla.lora_group_fwd(d["gdesc"], d["X"], d["W"], d["A"], d["B"], d["H"], d["U"], ws=self.ws,
                               ws_bytes=self.ws_bytes)
        elif "codes" in d:
            lla.lora_qlinear_fwd(d["desc"], d["X"], d["codes"], d["absmax"], d["codebook"], d["A"], d["B"],
                                 d["H"], d["U"], ws=self.ws, ws_bytes=self.ws_bytes)
        else:
            lla.lora_linear_fwd(d["desc"], d["X"], d["W"], d["A"], d["B"], d["H"], d["U"], ws=self.ws,
                                ws_bytes=self.ws_bytes)

    def bwd(self, d):
        lla = self.lla
        W = d.get("Wt", d.get("W"))          # W^T when the descriptor carries LORA_FLAG_W_TRANSPOSED
        if "g" in d:
            f = lla.lora_norm_group_bwd if "gdesc" in d else lla.lora_norm_linear_bwd
            f(d.get("gdesc") or d["desc"], NORM_EPS, d["dY"], d["X"], d["g"], W, d["A"], d["B"], d["U"],
              d["inv"], d["dX"], d["dA"], d["dB"], ws=self.ws, ws_bytes=self.ws_bytes)
        elif "gdesc" in d:
            lla.lora_group_bwd(d["gdesc"], d["dY"], d["X"], W, d["A"], d["B"], d["U"], d["dX"], d["dA"],
                               d["dB"], ws=self.ws, ws_bytes=self.ws_bytes)
        elif "codes" in d:
            lla.lora_qlinear_bwd(d["desc"], d["dY"], d["X"], d["codes"], d["absmax"], d["codebook"], d["A"],
                                 d["B"], d["U"], d["dX"], d["dA"], d["dB"], ws=self.ws, ws_bytes=self.ws_bytes)
        else:
            lla.lora_linear_bwd(d["desc"], d["dY"], d["X"], W, d["A"], d["B"], d["U"], d["dX"], d["dA"],
                                d["dB"], ws=self.ws, ws_bytes=self.ws_bytes)

    def step(self, layer):
        for li, d in enumerate(layer):
            self.current = li
            self.fwd(d)
        for li in reversed(range(len(layer))):
            self.current = li
            self.bwd(layer[li])


# ------------------------------------------------------------------ stand-alone HBM kernels
def event_time_us(torch, stream, run, reps=20):
    for _ in range(3):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3


def dequant_rate(lla, workloads, torch, dev, stream):
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
    us = event_time_us(torch, stream,
                       lambda: lla.lora_dequant4(codes, absmax, cb, N, K, lla.LORA_DTYPE_BF16, out, stream=stream))
    nbytes = N * K // 2 + 2 * (N * K // 64) + 2 * N * K
    gbps = nbytes / (us * 1e-6) / 1e9
    del codes, absmax, out
    return {"kernel": "dequant4_kernel (lora_dequant4, bf16 out)", "shape": [N, K], "bound": "hbm",
            "bytes_per_launch": nbytes, "avg_launch_us": round(us, 2), "achieved": round(gbps, 1),
            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}


def merge_rate(lla, torch, dev, stream, l):
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
    us = event_time_us(torch, stream, lambda: lla.lora_merge(desc, W, A, B, out, 1, stream=stream))
    nbytes = 4 * l.N * l.K + 2 * l.r * (l.K + l.N)
    gbps = nbytes / (us * 1e-6) / 1e9
    del W, A, B, out
    return {"kernel": "lora_merge (bf16)", "shape": [l.N, l.K, l.r], "bound": "hbm",
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


class HipEvents:
    """hipEvent_t handles from the HIP runtime the library itself uses (its
    symbols resolved through the library's handle)."""

    def __init__(self, lib):
        self.lib = lib
        self.made = []

    def _ok(self, err, what):
        if err != 0:
            raise RuntimeError(f"{what} failed with HIP error {err}")

    def create(self) -> int:
        ev = ctypes.c_void_p()
        self._ok(self.lib.hipEventCreate(ctypes.byref(ev)), "hipEventCreate")
        self.made.append(ev.value)
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        self._ok(self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)),
                 "hipEventElapsedTime")
        return ms.value

    def destroy_all(self):
        for e in self.made:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))
        self.made = []


def percentile(vals, q):
    v = sorted(vals)
    if not v:
        return None
    x = (len(v) - 1) * q
    lo, hi = int(x), min(int(x) + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (x - lo)


def parse_sclk_mhz(text):
    """Current shader clock from a DRM device's pp_dpm_sclk: the level marked
    with '*' (lines like '1: 2394Mhz *'); None when no level is marked."""
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            for tok in line.replace(":", " ").split():
                t = tok.lower()
                if t.endswith("mhz") and t[:-3].isdigit():
                    return int(t[:-3])
    return None


class ClockSampler:
    """Shader clock (pp_dpm_sclk) and socket power (hwmon power1_input, in
    microwatts) of the first DRM device that has both, read from sysfs every
    `period` seconds in a background thread while the steps run.  The chip
    sets its clock under load by its power limit, so these say what clock the
    measured rates were taken at."""

    def __init__(self, period=0.02):
        self.period, self.samples, self.sclk_path, self.power_path = period, [], None, None
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            sclk = os.path.join(dev, "pp_dpm_sclk")
            power = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_input")))
            if os.path.exists(sclk) and power:
                self.sclk_path, self.power_path = sclk, power[0]
                break
        self._stop = threading.Event()
        self._thread = None

    def _read(self):
        try:
            with open(self.sclk_path) as f:
                mhz = parse_sclk_mhz(f.read())
            with open(self.power_path) as f:
                watts = int(f.read().strip()) / 1e6
        except (OSError, ValueError):
            return None
        return time.perf_counter(), mhz, watts

    def _run(self):
        while not self._stop.is_set():
            s = self._read()
            if s is not None:
                self.samples.append(s)
            self._stop.wait(self.period)

    def start(self):
        if self.sclk_path is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self, t_from):
        """Medians and p10 / p90 over the samples taken from t_from on."""
        use = [(m, w) for t, m, w in self.samples if t >= t_from and m is not None]
        if not use:
            return None
        mhz, watts = [m for m, _ in use], [w for _, w in use]
        return {"sclk_mhz_p50": round(percentile(mhz, 0.5)),
                "sclk_mhz_p10_p90": [round(percentile(mhz, 0.1)), round(percentile(mhz, 0.9))],
                "power_w_p50": round(percentile(watts, 0.5)),
                "power_w_p10_p90": [round(percentile(watts, 0.1)), round(percentile(watts, 0.9))],
                "samples": len(use),
                "window": "second half of the device warm-up through the kernel-timer pass",
                "source": "sysfs pp_dpm_sclk (marked level), hwmon power1_input"}


def gemm_rooflines(units, kernel_us, traffic):
    """Roofline entries of the fused GEMMs from their measured mean durations
    (kernel_us: {(unit index, label): [launch durations in us]})."""
    out = []
    for (li, label), durs in sorted(kernel_us.items()):
        if not label.startswith("lora_gemm"):
            continue
        l = units[li]
        us = sum(durs) / len(durs)
        fl = gemm_flops(l, label)
        ach = fl / (us * 1e-6) / 1e12
        base = label.replace(" (split)", "")
        tr = traffic.get(base) if (traffic and len(units) == 1) else None
        out.append({"kernel": f"{label} ({l.name})", "bound": "mfma", "achieved": round(ach, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": tr, "avg_launch_us": round(us, 2), "launches_per_step": len(durs),
                    "flops_per_launch": fl, "algorithmic_bytes_per_launch": gemm_bytes(l, label)})
    return out


def norm_bytes(u, label: str) -> int:
    """Algorithmic HBM bytes of one launch of an RMSNorm row kernel.  The fold
    of g into A reads A [G r x K] and g and writes A diag(g); the preparation
    does that and also reads X once for 1/rms (M floats written); the
    input-gradient correction reads the GEMM's output and X, and 1/rms, and
    writes dX (bf16)."""
    M, K, R = u.M, u.K, u.G * u.r
    fold = 2 * R * K * 2 + 2 * K
    if label == "norm_prep":
        return 2 * M * K + 4 * M + fold
    if label == "norm_dx":
        return 3 * 2 * M * K + 4 * M
    return fold


def norm_rooflines(units, kernel_us):
    """HBM rooflines of the RMSNorm row kernels from their measured durations."""
    out = []
    for (li, label), durs in sorted(kernel_us.items()):
        if label not in NORM_KERNELS:
            continue
        u = units[li]
        us = sum(durs) / len(durs)
        b = norm_bytes(u, label)
        gbs = b / (us * 1e-6) / 1e9
        out.append({"kernel": f"{label} ({u.name})", "bound": "hbm", "achieved": round(gbs, 1),
                    "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBPS, 4),
                    "avg_launch_us": round(us, 2), "launches_per_step": len(durs),
                    "algorithmic_bytes_per_launch": b})
    return out


def vendor_gemm(torch, sets, wl, steps, stream):
    """The first linear's plain product X W^T by torch.matmul (hipBLASLt on
    ROCm) on the same rotating input sets: a reference for the fused forward
    GEMM, which also forms U and adds the rank-r term."""
    l = wl.linears[0]
    if l.quant4:
        return None
    outs = [torch.empty((l.M, l.N), dtype=torch.bfloat16, device=d["X"].device) for d in (s[0] for s in sets)]
    run = lambda i: torch.matmul(sets[i % len(sets)][0]["X"], sets[i % len(sets)][0]["W"].t(), out=outs[i % len(sets)])
    for i in range(5):
        run(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        run(i)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    fl = 2 * l.M * l.N * l.K
    return {"kernel": "torch.matmul(X, W.t()) (vendor GEMM, no LoRA terms)", "shape": [l.M, l.K, l.N],
            "avg_us": round(us, 2), "tflops": round(fl / (us * 1e-6) / 1e12, 1)}


def main(argv=None):
    args = parse(argv)
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
        for sh in wl.linears:
            d = workloads.device_inputs_torch(sh, dev, torch.bfloat16, seed=sh.seed * 100 + si)
            if sh.quant4:
                d.update(workloads.quantize4_torch(d.pop("W").float()))
            layer.append(d)
        layer = add_outputs(lla, torch, wl, share_inputs(wl, layer), dev)
        if args.norm:
            add_norm(lla, torch, wl, layer, dev, seed=7000 + 10 * si)
        if args.w_layout == "wt":
            add_wt(lla, torch, wl, layer)
        sets.append(layer)
    units = step_units(wl, args.grouped)
    if args.grouped:
        sets = [group_layer(lla, torch, wl, layer, units, dev) for layer in sets]
    stepper = Stepper(lla, torch, sets, dev)
    step = lambda i: stepper.step(sets[i % len(sets)])
    torch.cuda.synchronize()
    # device warm-up: real steps for a fixed wall time, until the clocks have
    # settled under load (before the tuner's probes and the counted warm-up)
    clock = ClockSampler().start()
    ramp_steps, ramp0 = 0, time.perf_counter()
    while time.perf_counter() - ramp0 < args.device_warmup_s:
        for _ in range(8):
            step(ramp_steps)
            ramp_steps += 1
        torch.cuda.synchronize()
    ramp_s = time.perf_counter() - ramp0
    tuned = {}
    if args.tune:
        for u, d in zip(units, sets[0]):
            if "gdesc" in d or "g" in d:
                continue                      # grouped and norm calls keep the built-in rules
            wargs = (dict(Wq=d["codes"], absmax=d["absmax"], codebook=d["codebook"]) if "codes" in d
                     else dict(W=d["W"]))
            # the tuner runs both directions with one W: its descriptor without the W^T flag
            tdesc = dataclasses.replace(d["desc"], flags=d["desc"].flags & ~lla.LORA_FLAG_W_TRANSPOSED)
            tuned[u.name] = lla.lora_tune_linear(tdesc, d["X"], d["A"], d["B"], d["H"], d["U"], d["dY"], d["dX"],
                                                 d["dA"], d["dB"], ws=stepper.ws, ws_bytes=stepper.ws_bytes, **wargs)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    run = step
    if args.graph:
        graphs = []
        for si in range(len(sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(si)
            graphs.append(g)
        torch.cuda.synchronize()
        run = lambda i: graphs[i % len(graphs)].replay()
        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)

    # 1. the timed region holds only the steps themselves
    t_start, t_end = mk(), mk()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        run(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # 1b. warm operands: the same K steps on one input set (its operands stay in
    # the Infinity Cache between steps when they fit), for comparison only
    w_start, w_end = mk(), mk()
    w_start.record(stream)
    for i in range(args.steps):
        run(0)
    w_end.record(stream)
    torch.cuda.synchronize()
    warm_ms_step = w_start.elapsed_time(w_end) / args.steps

    # 2. the same steps with events attached to every kernel's dispatch
    hev = HipEvents(lla.load())
    records = []          # (step, linear index, kernel label, start event, stop event)
    cur_step = [0]

    def timer(kernel, _stream):
        a, b = hev.create(), hev.create()
        records.append((cur_step[0], stepper.current, kernel, a, b))
        return a, b

    lla.lora_set_kernel_timer(timer)
    try:
        torch.cuda.synchronize()
        for i in range(args.steps):
            cur_step[0] = i
            step(i)
        torch.cuda.synchronize()
    finally:
        lla.lora_set_kernel_timer(None)
        clock.stop()
    kernel_us = {}
    first = {}
    for si, li, kernel, a, b in records:
        kernel_us.setdefault((li, kernel), []).append(hev.elapsed_ms(a, b) * 1e3)
        first.setdefault(si, (a, b))
    last = {}
    for si, li, kernel, a, b in records:
        last[si] = b
    step_ms = [hev.elapsed_ms(first[i][0], last[i]) for i in range(args.steps)]
    timer_ms_step = hev.elapsed_ms(first[0][0], last[args.steps - 1]) / args.steps
    hev.destroy_all()

    flops = wl.flops()
    tflops = flops / (ms_step * 1e-3) / 1e12
    tokens_s = wl.tokens / (ms_step * 1e-3)

    per_linear = []
    for li, u in enumerate(units):
        ks = {k: round(sum(v) / len(v), 2) for (i, k), v in kernel_us.items() if i == li}
        per_linear.append({"name": u.name, "kernel_us": ks})

    gemms = gemm_rooflines(units, kernel_us, load_traffic(wl.name, args.w_layout) if not args.norm else None)
    # dominant kernel: the GEMM with the largest measured time per step
    dominant = max(gemms, key=lambda g: g["avg_launch_us"] * g["launches_per_step"] / args.steps)
    p10, p50, p90 = (percentile(step_ms, q) for q in (0.1, 0.5, 0.9))

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "device_warmup": {"seconds": round(ramp_s, 3), "steps": ramp_steps},
        "clock": clock.summary(ramp0 + ramp_s / 2),
        "warm_operands": {"ms_per_step": round(warm_ms_step, 4),
                          "value": round(wl.flops() / (warm_ms_step * 1e-3) / 1e12, 2),
                          "note": "one input set reused every step (the headline value rotates input sets)"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "launch": "hip_graph_replay" if args.graph else "eager",
        "data": "synthetic (seeded on-device normal draws; no dataset or checkpoint)",
        "config": {"workload": wl.name, "linears": [[l.name, l.M, l.K, l.N, l.r, l.alpha] for l in wl.linears],
                   "input_sets": args.input_sets, "description": wl.description,
                   "calls": [u.name for u in units],
                   "rmsnorm_in_front": [u.name for u in units if behind_norm(wl.linears[u.members[0]].name)]
                   if args.norm else [],
                   "backward_weight": ("W^T [K, N] of the frozen weight, transposed once before timing"
                                       if args.w_layout == "wt" else "W [N, K]")},
        "tokens_per_s": round(tokens_s, 1), "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "step_ms_p10_p50_p90": [round(p10, 4), round(p50, 4), round(p90, 4)],
        "timed_kernels_ms_per_step": round(timer_ms_step, 4),
        "algorithmic_gflop_per_step": round(flops / 1e9, 3), "wall_s_timed": round(wall, 3),
        "per_linear": per_linear,
        "tuned": tuned if args.tune else None,
        "roofline": dict(dominant),
        "gemm_rooflines": gemms,
    }
    if args.norm:
        out["norm_rooflines"] = norm_rooflines(units, kernel_us)
    if args.vendor_gemm:
        out["vendor_gemm"] = vendor_gemm(torch, sets, wl, args.steps, stream)
    if not args.no_dequant:
        out["hbm_kernels"] = [dequant_rate(lla, workloads, torch, dev, stream),
                              merge_rate(lla, torch, dev, stream, max(wl.linears, key=lambda l: l.N * l.K))]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
