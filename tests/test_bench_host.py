"""Host logic of bench.py (no GPU): the one-GPU contract, the FLOP and byte
counts behind `value` and `roofline`, and the counter-CSV arithmetic behind
`roofline.traffic`."""
import argparse
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert p.returncode == 2
    assert "exactly one GPU" in json.loads(p.stdout.strip().splitlines()[-1])["error"]


@pytest.mark.parametrize("name", ["attn_proj_4096", "mlp_11008", "decoder_layer_r64", "qlora_28672"])
def test_fwd_plus_bwd_flops_are_the_algorithmic_count(name):
    """fwd (2MNK + 2Mr(K+N)) + bwd (2MNK + 4Mr(K+N)) = 4MNK + 6Mr(K+N) per linear."""
    wl = workloads.workload(name)
    assert sum(bench.fwd_flops(l) + bench.bwd_flops(l) for l in wl.linears) == wl.flops()
    for l in wl.linears:
        assert l.flops() == 4 * l.M * l.N * l.K + 6 * l.M * l.r * (l.K + l.N)


def test_forward_bytes():
    l = workloads.workload("attn_proj_4096").linears[0]
    M, K, N, r = l.M, l.K, l.N, l.r
    assert bench.fwd_bytes(l) == 2 * M * K + 2 * N * K + 2 * M * N + 2 * r * (K + N) + 4 * M * r
    q = workloads.workload("qlora_28672").linears[0]
    # 4-bit W: half a byte per code plus one fp16 absmax per 64 weights
    w4 = q.N * q.K // 2 + 2 * (q.N * q.K // 64)
    assert bench.fwd_bytes(q) == 2 * q.M * q.K + w4 + 2 * q.M * q.N + 2 * q.r * (q.K + q.N) + 4 * q.M * q.r


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_from_counter_csvs(tmp_path, monkeypatch):
    """Counters are averaged over each GEMM's dispatches and scaled by what the
    same counter reads for the calibration copy of known size."""
    fwd = "void lora::lora_gemm<false, 16, false, false, false>(lora::GemmArgs)"
    bwd = "void lora::lora_gemm<true, 16, false, false, false>(lora::GemmArgs)"
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"
    copy_kib = bench.COPY_BYTES / 1024
    _write_counters(tmp_path / "bench_FETCH_SIZE_counter_collection.csv",
                    [(fwd, "FETCH_SIZE", 1000.0), (fwd, "FETCH_SIZE", 3000.0), (bwd, "FETCH_SIZE", 5000.0)])
    _write_counters(tmp_path / "bench_WRITE_SIZE_counter_collection.csv",
                    [(fwd, "WRITE_SIZE", 500.0), (bwd, "WRITE_SIZE", 700.0), ("grad_final", "WRITE_SIZE", 9e9)])
    _write_counters(tmp_path / "copy_FETCH_SIZE_counter_collection.csv", [(neg, "FETCH_SIZE", copy_kib / 2)])
    _write_counters(tmp_path / "copy_WRITE_SIZE_counter_collection.csv", [(neg, "WRITE_SIZE", copy_kib)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(out))
    bench.write_traffic(argparse.Namespace(traffic_from=str(tmp_path), workload="attn_proj_4096", w_layout="wt"))
    t = json.load(open(out))
    f, b = t["kernels"][bench.GEMM_FWD], t["kernels"][bench.GEMM_DX]
    assert f["fetch_kib_per_dispatch"] == 2000.0 and f["write_kib_per_dispatch"] == 500.0
    assert b["fetch_kib_per_dispatch"] == 5000.0 and b["write_kib_per_dispatch"] == 700.0
    assert t["copy_fetch_factor"] == 0.5 and t["copy_write_factor"] == 1.0
    assert f["hbm_read_bytes_per_dispatch"] == 2000 * 1024 * 2
    assert f["hbm_write_bytes_per_dispatch"] == 500 * 1024
    assert t["kernel_source_hash"] == bench.kernel_source_hash()
    assert bench.load_traffic("attn_proj_4096") == {bench.GEMM_FWD: 2000 * 2048 + 500 * 1024,
                                                   bench.GEMM_DX: 5000 * 2048 + 700 * 1024}
    # ... only for the backward weight layout they were taken with
    assert bench.load_traffic("attn_proj_4096", "w") is None
    # ... and only while the GEMM's sources are unchanged
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic("attn_proj_4096") is None


def test_gemm_flops_and_bytes():
    """Per-launch algorithmic counts of the two GEMMs: the in-tile forms also
    carry the rank-r product (U = X A^T, V = dY B); their sum with the
    adapter-gradient products is the layer's 4MNK + 6Mr(K+N)."""
    l = workloads.workload("attn_proj_4096").linears[0]
    M, K, N, r = l.M, l.K, l.N, l.r
    assert bench.gemm_flops(l, bench.GEMM_FWD) == 2 * M * N * K + 2 * M * N * r + 2 * M * r * K
    assert bench.gemm_flops(l, bench.GEMM_DX) == 2 * M * N * K + 2 * M * K * r + 2 * M * r * N
    grads = 2 * M * r * K + 2 * M * N * r      # dA = s V^T X, dB = s dY^T U
    assert bench.gemm_flops(l, bench.GEMM_FWD) + bench.gemm_flops(l, bench.GEMM_DX) + grads == l.flops()
    # r > 16: the rank-r product comes from the streamed pass, not the GEMM
    d = workloads.workload("decoder_layer_r64").linears[0]
    assert bench.gemm_flops(d, bench.GEMM_FWD) == 2 * d.M * d.N * d.K + 2 * d.M * d.N * d.r
    assert bench.gemm_flops(d, bench.GEMM_DX + " (split)") == 2 * d.M * d.K * d.N + 2 * d.M * d.K * d.r
    assert bench.gemm_bytes(l, bench.GEMM_FWD) == bench.fwd_bytes(l)
    assert bench.gemm_bytes(l, bench.GEMM_DX) == (2 * M * N + 2 * N * K + 2 * M * K + 2 * r * (K + N) + 4 * M * r
                                                  + 8 * r * M)


def test_percentile_and_input_sharing():
    assert bench.percentile([4.0, 1.0, 3.0, 2.0, 5.0], 0.5) == 3.0
    assert bench.percentile([1.0, 2.0], 0.1) == 1.1
    wl = workloads.workload("decoder_layer_r64")
    layer = [{"X": object()} for _ in wl.linears]
    xs = [d["X"] for d in layer]
    bench.share_inputs(wl, layer)
    names = [l.name.split("_")[-1] for l in wl.linears]
    got = dict(zip(names, (d["X"] for d in layer)))
    assert got["q"] is got["k"] is got["v"] is xs[0]
    assert got["gate"] is got["up"] is xs[names.index("gate")]
    assert got["o"] is xs[names.index("o")] and got["down"] is xs[names.index("down")]


def test_missing_counters_are_an_error(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(tmp_path / "t.json"))
    with pytest.raises(SystemExit):
        bench.write_traffic(argparse.Namespace(traffic_from=str(tmp_path), workload="attn_proj_4096", w_layout="wt"))


def test_grouped_units_and_counts():
    """--grouped: q/k/v and gate/up become one call each; the GEMM counts of a
    group add up to its members' (the same dense and rank-r products)."""
    wl = workloads.workload("decoder_layer_r64")
    units = bench.step_units(wl, True)
    assert [u.name for u in units] == ["decoder_q+decoder_k+decoder_v", "decoder_o", "decoder_gate+decoder_up",
                                       "decoder_down"]
    assert [u.G for u in units] == [3, 1, 2, 1] and units[0].N == 4096 + 1024 + 1024
    assert [u.name for u in bench.step_units(wl, False)] == [l.name for l in wl.linears]
    for u in units:
        mem = [wl.linears[i] for i in u.members]
        for label in (bench.GEMM_FWD, bench.GEMM_DX):
            assert bench.gemm_flops(u, label) == sum(bench.gemm_flops(m, label) for m in mem)


def test_norm_selection_and_row_kernel_bytes():
    """--norm puts the RMSNorm in front of the linears that read a normalised
    input (q/k/v, gate/up, the single 4096 projection), not o or down; the row
    kernels' algorithmic bytes: 1/rms reads X once, the correction reads the
    GEMM output and X and writes dX, the A fold reads and writes G r x K."""
    dec = [l.name for l in workloads.workload("decoder_layer_r64").linears]
    assert [n for n in dec if bench.behind_norm(n)] == ["decoder_q", "decoder_k", "decoder_v", "decoder_gate",
                                                        "decoder_up"]
    assert bench.behind_norm("attn_proj_4096")
    assert not any(bench.behind_norm(l.name) for l in workloads.workload("qlora_28672").linears)
    u = bench.Unit("qkv", 4096, 4096, 6144, 64, 16.0, 3)
    fold = 4 * 192 * 4096 + 2 * 4096
    assert bench.norm_bytes(u, "norm_fold") == fold
    assert bench.norm_bytes(u, "norm_prep") == 2 * 4096 * 4096 + 4 * 4096 + fold
    assert bench.norm_bytes(u, "norm_dx") == 6 * 4096 * 4096 + 4 * 4096
    ks = {(0, "norm_prep"): [10.0, 10.0], (0, "norm_dx"): [20.0], (0, "lora_gemm forward"): [100.0]}
    rows = bench.norm_rooflines([u], ks)
    assert [r["kernel"] for r in rows] == ["norm_dx (qkv)", "norm_prep (qkv)"]
    assert rows[1]["achieved"] == pytest.approx((2 * 4096 * 4096 + 4 * 4096 + fold) / 10e-6 / 1e9, rel=1e-3)


def test_clock_sampler_parsing_and_summary():
    """pp_dpm_sclk's marked level is the current clock; the summary keeps only the
    samples from the given time on and reports medians and p10 / p90."""
    assert bench.parse_sclk_mhz("S: 101Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == 101
    assert bench.parse_sclk_mhz("S: 101Mhz\n0: 500Mhz\n1: 2394Mhz *\n") == 2394
    assert bench.parse_sclk_mhz("0: 500Mhz\n1: 2400Mhz\n") is None
    c = bench.ClockSampler()
    c.samples = [(0.0, 157, 253.0), (1.0, 2100, 1340.0), (2.0, 2130, 1350.0), (3.0, 2140, 1360.0),
                 (4.0, None, 1000.0)]
    s = c.summary(1.0)
    assert s["samples"] == 3
    assert s["sclk_mhz_p50"] == 2130 and s["power_w_p50"] == 1350
    assert s["sclk_mhz_p10_p90"] == [2106, 2138]
    assert c.summary(5.0) is None
