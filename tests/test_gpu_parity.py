"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Graded check: the oracle runs on the float32 draws, the GPU on their bf16
images (bf16 mode) or on the draws themselves (float32 checking mode); the
bound is max|err|/max|ref| <= 1e-2 (bf16) or 1e-5 (float32).  A diagnostic
check runs the oracle on exactly the values the GPU received: then the only
error left is the final bf16 rounding of each output: bf16 keeps 8
significant bits, so that rounding costs at most 2^-8 of the output's own
magnitude, hence <= 2^-8 * max|ref| (plus float32 accumulation error).
The graded bound is asserted on the workload shapes; the ragged and
degenerate shapes (e.g. one token, rank 1) use the diagnostic bound, because
the bf16 rounding of a few inputs can by itself move a short sum by >1 %.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import (BF16_TOL, F32_TOL, device_inputs, host_view, rel_err, run_linear, to_dev,
                         to_np)

pytestmark = pytest.mark.gpu

TOL = {"bf16": BF16_TOL, "f32": F32_TOL}
DIAG = {"bf16": 4e-3, "f32": F32_TOL}   # 2^-8 = 3.906e-3


def oracle_all(inp, s, rows=None):
    X, W, A, B, dY = inp["X"], inp["W"], inp["A"], inp["B"], inp["dY"]
    Xr = X if rows is None else X[rows]
    dYr = dY if rows is None else dY[rows]
    H, U = oracle.forward(Xr, W, A, B, s)
    dX = oracle.backward_dx(dYr, W, A, B, s)
    dA, dB = oracle.backward_lora(dY, X, A, B, s)
    return {"H": H, "U": U, "dX": dX, "dA": dA, "dB": dB}


def check(got, ref, tol, rows=None, keys=("H", "U", "dX", "dA", "dB"), label=""):
    errs = {}
    for k in keys:
        if k not in got:
            continue
        g = got[k] if rows is None or k in ("dA", "dB") else got[k][rows]
        errs[k] = rel_err(g, ref[k])
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, f"{label} errors {errs} exceed {tol}"
    return errs


def shape(M, K, N, r, alpha=32.0, seed=7):
    return workloads.LinearShape("case", M, K, N, r, alpha, seed)


# ----------------------------------------------------------------------------- tiny
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tiny_workload(dtype):
    sh = workloads.workload("tiny").linears[0]
    inp = workloads.make_linear_inputs(sh)
    got = run_linear(inp, sh.r, sh.alpha, dtype)
    check(got, oracle_all(inp, sh.scale), TOL[dtype], label="graded")
    check(got, oracle_all(host_view(inp, dtype), sh.scale), DIAG[dtype], label="diagnostic")


# ---------------------------------------------------------------- ragged / rank sweep
RAGGED = [
    (300, 136, 264, 5), (1, 8, 8, 1), (257, 520, 72, 16), (130, 64, 1000, 24),
    (513, 264, 256, 48), (64, 128, 128, 64), (200, 192, 136, 100), (96, 256, 264, 128),
    (520, 72, 520, 8), (33, 2056, 40, 3),
    (300, 200, 1000, 24),    # r > 16 with few output tiles: forward in 2 and dX in 8 contraction slices
    (4352, 320, 4136, 24),   # 289 forward tiles, ragged in both directions; dX (34 tiles) in 8 slices
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,N,r", RAGGED)
def test_ragged_shapes(M, K, N, r, dtype):
    sh = shape(M, K, N, r, seed=M * 7 + K + N + r)
    inp = workloads.make_linear_inputs(sh)
    got = run_linear(inp, r, sh.alpha, dtype)
    check(got, oracle_all(host_view(inp, dtype), sh.scale), DIAG[dtype], label=f"{(M, K, N, r)} diagnostic")


@pytest.mark.parametrize("M,K,N,r", [(64, 1 << 21, 64, 8), (64, 64, 1 << 21, 8), (72, (1 << 21) - 8, 40, 16)])
def test_maximum_dims(M, K, N, r):
    """K or N at the descriptor's bound 2^21 (the largest per-tile buffer offsets;
    with one output tile the contraction runs split into slices), bf16."""
    sh = shape(M, K, N, r, seed=M + r + (K >> 10) + (N >> 10))
    print(f"max dims M={M} K={K} N={N} r={r}", flush=True)
    inp = workloads.make_linear_inputs(sh)
    got = run_linear(inp, r, sh.alpha, "bf16")
    check(got, oracle_all(host_view(inp, "bf16"), sh.scale), DIAG["bf16"], label=f"{(M, K, N, r)} diagnostic")


# ------------------------------------------------------------------- special cases
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_b_zero_is_plain_linear(dtype):
    sh = shape(192, 264, 320, 8)
    inp = workloads.make_linear_inputs(sh)
    inp["B"] = np.zeros_like(inp["B"])
    got = run_linear(inp, sh.r, sh.alpha, dtype)
    ref = oracle_all(host_view(inp, dtype), sh.scale)
    assert not np.any(got["dA"]), "dA must be exactly zero when B = 0"
    assert np.any(got["dB"])
    check(got, ref, DIAG[dtype], keys=("H", "dX", "dB"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_a_zero_and_s_zero(dtype):
    sh = shape(160, 136, 200, 16)
    inp = workloads.make_linear_inputs(sh)
    a0 = dict(inp, A=np.zeros_like(inp["A"]))
    got = run_linear(a0, sh.r, sh.alpha, dtype)
    assert not np.any(got["dB"]) and not np.any(got["U"])
    check(got, oracle_all(host_view(a0, dtype), sh.scale), DIAG[dtype], keys=("H", "dX", "dA"))
    got0 = run_linear(inp, sh.r, 0.0, dtype)
    assert not np.any(got0["dA"]) and not np.any(got0["dB"])
    check(got0, oracle_all(host_view(inp, dtype), 0.0), DIAG[dtype], keys=("H", "dX"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_hot_probes_are_exact(dtype):
    """B = 0 and one-hot rows: each output is a single exact product, so bit-exact."""
    M, K, N, r = 300, 520, 264, 8
    sh = shape(M, K, N, r)
    inp = workloads.make_linear_inputs(sh)
    hv = host_view(inp, dtype)
    rng = np.random.default_rng(5)
    kk = rng.integers(0, K, size=M)
    nn = rng.integers(0, N, size=M)
    X = np.zeros((M, K), np.float32); X[np.arange(M), kk] = 1.0
    dY = np.zeros((M, N), np.float32); dY[np.arange(M), nn] = 1.0
    probe = dict(inp, X=X, dY=dY, B=np.zeros_like(inp["B"]))
    got = run_linear(probe, r, sh.alpha, dtype)
    W = hv["W"]
    np.testing.assert_array_equal(got["H"], W[:, kk].T)           # H[m, n] = W[n, k(m)]
    np.testing.assert_array_equal(got["dX"], W[nn, :])            # dX[m, k] = W[n(m), k]
    np.testing.assert_array_equal(got["U"], hv["A"][:, kk].T)     # U[m, j] = A[j, k(m)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deterministic(dtype):
    sh = shape(1000, 392, 520, 16)
    inp = workloads.make_linear_inputs(sh)
    dev = device_inputs(inp, dtype)
    a = run_linear(inp, sh.r, sh.alpha, dtype, dev_inputs=dev)
    b = run_linear(inp, sh.r, sh.alpha, dtype, dev_inputs=dev)
    for k in a:
        np.testing.assert_array_equal(a[k].view(np.uint32), b[k].view(np.uint32), err_msg=k)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_accumulate_flag(dtype):
    import lora_linear_layer_amd as lla
    sh = shape(200, 136, 144, 8)
    inp = workloads.make_linear_inputs(sh)
    rng = np.random.default_rng(9)
    dA0 = rng.standard_normal(inp["A"].shape).astype(np.float32)
    dB0 = rng.standard_normal(inp["B"].shape).astype(np.float32)
    got = run_linear(inp, sh.r, sh.alpha, dtype, flags=lla.LORA_FLAG_ACCUM_GRADS, grads_init=(dA0, dB0))
    ref = oracle_all(host_view(inp, dtype), sh.scale)
    hv0 = host_view({"X": dA0, "W": dB0}, dtype)
    ref["dA"] = ref["dA"] + hv0["X"]
    ref["dB"] = ref["dB"] + hv0["W"]
    check(got, ref, DIAG[dtype], keys=("dA", "dB"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("r", [8, 100])
def test_recompute_u_and_skip_dx(dtype, r):
    sh = shape(264, 200, 136, r)
    inp = workloads.make_linear_inputs(sh)
    ref = oracle_all(host_view(inp, dtype), sh.scale)
    got = run_linear(inp, r, sh.alpha, dtype, save_u=False)
    check(got, ref, DIAG[dtype], keys=("H", "dX", "dA", "dB"))
    got = run_linear(inp, r, sh.alpha, dtype, want_dx=False)
    check(got, ref, DIAG[dtype], keys=("H", "dA", "dB"))


# ---------------------------------------------------------------- full-size workloads
FULL = [("attn_proj_4096", 0)] + [("mlp_11008", i) for i in range(3)] + \
       [("decoder_layer_r64", i) for i in range(7)]


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("wl,idx", FULL)
def test_full_size(wl, idx, dtype):
    """Every element of H, U, dX, dA and dB at the workload's full size."""
    sh = workloads.workload(wl).linears[idx]
    inp = workloads.make_linear_inputs(sh)
    print(f"full-size {sh.name} M={sh.M} K={sh.K} N={sh.N} r={sh.r} {dtype}", flush=True)
    got = run_linear(inp, sh.r, sh.alpha, dtype)
    ref = oracle_all(inp, sh.scale)
    errs = check(got, ref, TOL[dtype], label=f"{sh.name} graded")
    print(f"  graded errors {errs}", flush=True)


@pytest.mark.slow
@pytest.mark.parametrize("wl,idx", FULL)
def test_full_size_w_transposed(wl, idx):
    """The backward with the frozen weight given as W^T (LORA_FLAG_W_TRANSPOSED,
    the layout bench.py times): every element against the oracle."""
    import lora_linear_layer_amd as lla
    sh = workloads.workload(wl).linears[idx]
    inp = workloads.make_linear_inputs(sh)
    print(f"full-size W^T {sh.name} M={sh.M} K={sh.K} N={sh.N} r={sh.r}", flush=True)
    got = run_linear(inp, sh.r, sh.alpha, "bf16", flags=lla.LORA_FLAG_W_TRANSPOSED)
    ref = oracle_all(inp, sh.scale)
    errs = check(got, ref, TOL["bf16"], label=f"{sh.name} W^T graded")
    print(f"  graded errors {errs}", flush=True)


@pytest.mark.slow
def test_input_over_2gb():
    """X of 262208 x 4096 bf16 (2.15 GB: its last 64 rows lie past 2^31 bytes),
    r = 32, so U = X A^T comes from the streamed pass whose loads address X
    from each 128-row block; every element of H, U, dX, dA and dB against the
    oracle on the exact bf16 inputs (rows chunked to bound host memory)."""
    M, K, N, r = (1 << 30) // 4096 + 64, 4096, 64, 32
    sh = shape(M, K, N, r, alpha=16.0, seed=2048)
    print(f"input over 2 GB: M={M} K={K} N={N} r={r}", flush=True)
    inp = workloads.make_linear_inputs(sh)
    hv = host_view(inp, "bf16")
    del inp
    got = run_linear(hv, r, sh.alpha, "bf16")
    print("  GPU done", flush=True)
    X, W, A, B, dY, s = hv["X"], hv["W"], hv["A"], hv["B"], hv["dY"], sh.scale
    num = {k: 0.0 for k in ("H", "U", "dX")}
    den = dict(num)
    step = 1 << 16
    for m0 in range(0, M, step):
        Hc, Uc = oracle.forward(X[m0:m0 + step], W, A, B, s)
        dXc = oracle.backward_dx(dY[m0:m0 + step], W, A, B, s)
        for k, ref in (("H", Hc), ("U", Uc), ("dX", dXc)):
            num[k] = max(num[k], float(np.abs(got[k][m0:m0 + step] - ref).max()))
            den[k] = max(den[k], float(np.abs(ref).max()))
    errs = {k: num[k] / den[k] for k in num}
    dA, dB = oracle.backward_lora(dY, X, A, B, s)
    errs["dA"] = rel_err(got["dA"], dA)
    errs["dB"] = rel_err(got["dB"], dB)
    # rows past the 2 GB mark on their own (the blocks the old single resource read as zeros)
    tail = slice((1 << 30) // K, M)
    Ht, Ut = oracle.forward(X[tail], W, A, B, s)
    errs["U past 2 GB"] = rel_err(got["U"][tail], Ut)
    errs["H past 2 GB"] = rel_err(got["H"][tail], Ht)
    print(f"  diagnostic errors {errs}", flush=True)
    bad = {k: e for k, e in errs.items() if not e <= DIAG["bf16"]}
    assert not bad, f"errors {errs} exceed {DIAG['bf16']}"


# ---------------------------------------------------------------------- 4-bit path
def q_inputs(M, K, N, r, seed):
    sh = workloads.LinearShape("q", M, K, N, r, 32.0, seed, True)
    return sh, workloads.make_qlora_inputs(sh)


def q_oracle_inputs(inp, dtype):
    d = dict(inp)
    d["W"] = oracle.dequant4(inp["codes"], inp["absmax"], oracle.codebook4(), out="bf16" if dtype == "bf16" else "f32")
    return d


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dequant4_bit_exact(out):
    import lora_linear_layer_amd as lla
    _, inp = q_inputs(8, 1024, 264, 4, 31)
    N, K = 264, 1024
    dev = device_inputs(inp, "bf16", quant=True)
    tdt = torch.bfloat16 if out == "bf16" else torch.float32
    W = torch.empty((N, K), dtype=tdt, device="cuda")
    lla.lora_dequant4(dev["codes"], dev["absmax"], dev["codebook"], N, K,
                      lla.LORA_DTYPE_BF16 if out == "bf16" else lla.LORA_DTYPE_F32, W)
    torch.cuda.synchronize()
    ref = oracle.dequant4(inp["codes"], inp["absmax"], oracle.codebook4(), out=out)
    np.testing.assert_array_equal(to_np(W).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dequant4_bit_exact_grid_stride(out):
    """4104 x 8192 weights (4.2 M groups of 8): every thread takes the four-groups-in-flight
    path of the grid-stride loop once and some take the remainder path after it."""
    import lora_linear_layer_amd as lla
    N, K = 4104, 8192
    rng = np.random.default_rng(4104)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    absmax = (rng.random((N, K // 64)) * 0.08 + 0.01).astype(np.float16)
    cb = workloads.codebook4_f32()
    tdt = torch.bfloat16 if out == "bf16" else torch.float32
    W = torch.empty((N, K), dtype=tdt, device="cuda")
    lla.lora_dequant4(torch.from_numpy(codes).cuda(), torch.from_numpy(absmax.view(np.int16)).cuda(),
                      torch.from_numpy(cb).cuda(), N, K, lla.LORA_DTYPE_BF16 if out == "bf16" else lla.LORA_DTYPE_F32, W)
    torch.cuda.synchronize()
    ref = oracle.dequant4(codes, absmax, cb, out=out)
    np.testing.assert_array_equal(to_np(W).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,N,r", [(300, 256, 264, 16), (64, 1024, 136, 8), (130, 192, 520, 100),
                                     (4352, 320, 4136, 24)])   # 289 forward tiles: the last 33 in 2 slices
def test_qlinear_parity(M, K, N, r, dtype):
    sh, inp = q_inputs(M, K, N, r, M + K + N)
    got = run_linear(inp, r, sh.alpha, dtype, quant=True)
    ref_in = q_oracle_inputs(inp, dtype)
    check(got, oracle_all(host_view(ref_in, dtype) | {"W": ref_in["W"]}, sh.scale), DIAG[dtype], label="diag")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qlinear_one_hot_exact(dtype):
    M, K, N, r = 200, 512, 264, 16
    sh, inp = q_inputs(M, K, N, r, 41)
    Wd = q_oracle_inputs(inp, dtype)["W"]
    rng = np.random.default_rng(6)
    kk = rng.integers(0, K, size=M)
    nn = rng.integers(0, N, size=M)
    X = np.zeros((M, K), np.float32); X[np.arange(M), kk] = 1.0
    dY = np.zeros((M, N), np.float32); dY[np.arange(M), nn] = 1.0
    probe = dict(inp, X=X, dY=dY, B=np.zeros_like(inp["B"]))
    got = run_linear(probe, r, sh.alpha, dtype, quant=True)
    np.testing.assert_array_equal(got["H"], Wd[:, kk].T)
    np.testing.assert_array_equal(got["dX"], Wd[nn, :])


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qlora_full_size(dtype):
    """Every element of H, U, dX, dA and dB of the 4-bit layer at full size."""
    sh = workloads.workload("qlora_28672").linears[0]
    inp = workloads.make_qlora_inputs(sh)
    print(f"full-size {sh.name} {dtype}", flush=True)
    got = run_linear(inp, sh.r, sh.alpha, dtype, quant=True)
    ref_in = q_oracle_inputs(inp, dtype)
    errs = check(got, oracle_all(ref_in, sh.scale), TOL[dtype], label="graded")
    print(f"  graded errors {errs}", flush=True)


def all_absmax_patterns():
    """Codes and absmax covering every fp16 bit pattern (row n has absmax bits n)
    with every code (weight k of a row has code k % 16)."""
    N, K = 1 << 16, 64
    k = np.arange(K)
    row = (k[0::2] % 16) | ((k[1::2] % 16) << 4)
    codes = np.broadcast_to(row.astype(np.uint8), (N, K // 2)).copy()
    absmax = np.arange(N, dtype=np.uint32).astype(np.uint16).reshape(N, 1)
    return codes, absmax, N, K


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dequant4_every_absmax_pattern(out):
    """All 65536 fp16 absmax bit patterns (+-0, subnormals, normals, negative
    values, +-inf, NaN) times all 16 codes through the stand-alone
    dequantisation: bit-exact against the oracle; where the oracle gives NaN
    (absmax NaN) the GPU must give NaN too (its payload is not specified)."""
    import lora_linear_layer_amd as lla
    codes, absmax, N, K = all_absmax_patterns()
    cb = workloads.codebook4_f32()
    tdt = torch.bfloat16 if out == "bf16" else torch.float32
    W = torch.empty((N, K), dtype=tdt, device="cuda")
    lla.lora_dequant4(torch.from_numpy(codes).cuda(), torch.from_numpy(absmax.view(np.int16)).cuda(),
                      torch.from_numpy(cb).cuda(), N, K, lla.LORA_DTYPE_BF16 if out == "bf16" else lla.LORA_DTYPE_F32, W)
    torch.cuda.synchronize()
    got = to_np(W)
    ref = oracle.dequant4(codes, absmax, cb, out=out)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 1023 * K                     # 0x7C01..0x7FFF and 0xFC01..0xFFFF
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.signbit(got[0]).tolist() == [bool(c < 0) for c in cb[np.arange(K) % 16]]   # absmax +0: signed zeros


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qlinear_one_hot_edge_absmax(dtype):
    """The dequantisation inside the fused 4-bit GEMMs with edge absmax values
    (+-0, the smallest and largest subnormals, the smallest normal, negative
    values, the largest finite fp16): B = 0 and one-hot rows make each output
    one weight, which must equal the oracle's dequantised value exactly."""
    M, K, N, r = 192, 512, 264, 16
    sh, inp = q_inputs(M, K, N, r, 43)
    edge = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x8400, 0x3C00, 0xBC00, 0x7BFF, 0xFBFF,
                     0x2E66], dtype=np.uint16)
    rng = np.random.default_rng(8)
    inp["absmax"] = edge[rng.integers(0, edge.size, size=inp["absmax"].shape)].view(np.float16)
    Wd = q_oracle_inputs(inp, dtype)["W"]
    kk = rng.integers(0, K, size=M)
    nn = rng.integers(0, N, size=M)
    X = np.zeros((M, K), np.float32); X[np.arange(M), kk] = 1.0
    dY = np.zeros((M, N), np.float32); dY[np.arange(M), nn] = 1.0
    probe = dict(inp, X=X, dY=dY, B=np.zeros_like(inp["B"]))
    got = run_linear(probe, r, sh.alpha, dtype, quant=True)
    np.testing.assert_array_equal(got["H"], Wd[:, kk].T)
    np.testing.assert_array_equal(got["dX"], Wd[nn, :])


@pytest.mark.parametrize("r,want_dx", [(8, True), (100, False)])
def test_workspace_garbage_and_reuse(r, want_dx):
    """The adapter-gradient pass keeps per-tile counters in the workspace: the
    backward clears them itself, so a workspace full of 0xFF bytes and a second
    backward on the same workspace give the oracle's gradients, bit-identical
    between the two calls.  r = 8 with dX: V formed in the dX GEMM, which writes
    the rank planes and clears the counters; r = 100 without dX: the streamed V
    pass, two adapter-gradient launches (64 rank columns each)."""
    import lora_linear_layer_amd as lla
    sh = shape(520, 392, 264, r)
    inp = workloads.make_linear_inputs(sh)
    dd = device_inputs(inp, "bf16")
    desc = lla.Desc(sh.M, sh.K, sh.N, r, sh.alpha)
    ws = torch.full((lla.lora_linear_workspace_size(desc),), 0xFF, dtype=torch.uint8, device="cuda")
    H = torch.empty((sh.M, sh.N), dtype=torch.bfloat16, device="cuda")
    U = torch.empty((sh.M, r), dtype=torch.float32, device="cuda")
    lla.lora_linear_fwd(desc, dd["X"], dd["W"], dd["A"], dd["B"], H, U, ws=ws)
    outs = []
    for _ in range(2):
        dX = torch.empty((sh.M, sh.K), dtype=torch.bfloat16, device="cuda") if want_dx else None
        dA = torch.empty((r, sh.K), dtype=torch.bfloat16, device="cuda")
        dB = torch.empty((sh.N, r), dtype=torch.bfloat16, device="cuda")
        lla.lora_linear_bwd(desc, dd["dY"], dd["X"], dd["W"], dd["A"], dd["B"], U, dX, dA, dB, ws=ws)
        torch.cuda.synchronize()
        outs.append({"dA": to_np(dA), "dB": to_np(dB)} | ({"dX": to_np(dX)} if want_dx else {}))
    ref = oracle_all(host_view(inp, "bf16"), sh.scale)
    check(outs[1], ref, DIAG["bf16"], keys=("dX", "dA", "dB"))
    for k in outs[0]:
        np.testing.assert_array_equal(outs[0][k].view(np.uint32), outs[1][k].view(np.uint32), err_msg=k)
