"""GPU parity of linears that share one input (lora_group_fwd / lora_group_bwd)
against the oracle's group_forward / group_backward.

Members are drawn like single linears (X shared: the first member's draw);
on the device they are stacked as the C ABI expects (W, B, H, dY by output
columns, A, U by rank rows).  Ragged member widths put member boundaries
inside output tiles; a one-member group must reproduce the plain entry points
bit for bit.  Bound: the diagnostic one (the oracle on exactly the bf16
inputs the GPU received), as for the other ragged shapes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import host_view, rel_err, run_linear, to_dev, to_np

pytestmark = pytest.mark.gpu

DIAG = 4e-3


def group_inputs(M, K, Ns, r, seed):
    """Per-member draws of make_linear_inputs; every member reads member 0's X."""
    mem = [workloads.make_linear_inputs(workloads.LinearShape(f"m{i}", M, K, n, r, 32.0, seed + i))
           for i, n in enumerate(Ns)]
    return {"X": mem[0]["X"], "W": [m["W"] for m in mem], "A": [m["A"] for m in mem],
            "B": [m["B"] for m in mem], "dY": [m["dY"] for m in mem]}


def bf16_view(g):
    out = {"X": host_view({"X": g["X"]}, "bf16")["X"]}
    for k in ("W", "A", "B", "dY"):
        out[k] = [host_view({"X": a}, "bf16")["X"] for a in g[k]]
    return out


def run_group(g, r, alpha, *, save_u=True, want_dx=True, flags=0, grads_init=None):
    import lora_linear_layer_amd as lla
    M, K = g["X"].shape
    Ns = tuple(w.shape[0] for w in g["W"])
    desc = lla.GroupDesc(M, K, Ns, r, alpha, flags=flags)
    bf = torch.bfloat16
    X = to_dev(g["X"], bf)
    W = to_dev(np.vstack(g["W"]), bf)
    A = to_dev(np.vstack(g["A"]), bf)
    B = to_dev(np.vstack(g["B"]), bf)
    dY = to_dev(np.hstack(g["dY"]), bf)
    N, R = sum(Ns), len(Ns) * r
    H = torch.empty((M, N), dtype=bf, device="cuda")
    U = torch.empty((M, R), dtype=torch.float32, device="cuda") if save_u else None
    dX = torch.empty((M, K), dtype=bf, device="cuda") if want_dx else None
    if grads_init is not None:
        dA, dB = to_dev(grads_init[0], bf), to_dev(grads_init[1], bf)
    else:
        dA = torch.empty((R, K), dtype=bf, device="cuda")
        dB = torch.empty((N, r), dtype=bf, device="cuda")
    lla.lora_group_fwd(desc, X, W, A, B, H, U)
    lla.lora_group_bwd(desc, dY, X, W, A, B, U, dX, dA, dB)
    torch.cuda.synchronize()
    cols = np.cumsum((0,) + Ns)
    out = {"H": [to_np(H)[:, cols[i]:cols[i + 1]] for i in range(len(Ns))],
           "dA": [to_np(dA)[i * r:(i + 1) * r] for i in range(len(Ns))],
           "dB": [to_np(dB)[cols[i]:cols[i + 1]] for i in range(len(Ns))]}
    if save_u:
        out["U"] = [to_np(U)[:, i * r:(i + 1) * r] for i in range(len(Ns))]
    if want_dx:
        out["dX"] = to_np(dX)
    return out


def group_errors(got, ref_in, s, keys=("H", "U", "dX", "dA", "dB")):
    outs = oracle.group_forward(ref_in["X"], ref_in["W"], ref_in["A"], ref_in["B"], s)
    dX, dAs, dBs = oracle.group_backward(ref_in["dY"], ref_in["X"], ref_in["W"], ref_in["A"], ref_in["B"], s)
    ref = {"H": [h for h, _ in outs], "U": [u for _, u in outs], "dX": dX, "dA": dAs, "dB": dBs}
    errs = {}
    for k in keys:
        if k not in got:
            continue
        if k == "dX":
            errs[k] = rel_err(got[k], ref[k])
        else:
            errs[k] = max(rel_err(a, b) for a, b in zip(got[k], ref[k]))
    return errs


GROUPS = [
    (300, 392, (264, 136, 520), 16),     # boundaries at 264 and 400: inside output tiles
    (257, 520, (72, 1000), 24),
    (130, 264, (64, 64, 64), 64),        # group rank 192 (one 192-column U pass); three members in one tile
    (513, 136, (1024, 256, 256), 64),    # q / k / v proportions
    (96, 256, (264, 264), 96),           # r > 64: dB of each member in a 64- and a 32-column problem
    (64, 1024, (8, 16, 8, 24, 8, 16, 8, 40), 8),   # eight narrow members
]


@pytest.mark.parametrize("M,K,Ns,r", GROUPS)
def test_group_parity(M, K, Ns, r):
    g = group_inputs(M, K, Ns, r, seed=M + K + r)
    print(f"group M={M} K={K} N={Ns} r={r}", flush=True)
    got = run_group(g, r, 32.0)
    errs = group_errors(got, bf16_view(g), 32.0 / r)
    print(f"  diagnostic errors {errs}", flush=True)
    assert all(e <= DIAG for e in errs.values()), errs


def test_group_recompute_u_skip_dx_and_accumulate():
    M, K, Ns, r = 200, 264, (136, 264), 32
    g = group_inputs(M, K, Ns, r, seed=5)
    hv = bf16_view(g)
    got = run_group(g, r, 16.0, save_u=False)
    assert all(e <= DIAG for e in group_errors(got, hv, 0.5, keys=("H", "dX", "dA", "dB")).values())
    got = run_group(g, r, 16.0, want_dx=False)
    assert all(e <= DIAG for e in group_errors(got, hv, 0.5, keys=("H", "U", "dA", "dB")).values())
    rng = np.random.default_rng(3)
    dA0 = rng.standard_normal((len(Ns) * r, K)).astype(np.float32)
    dB0 = rng.standard_normal((sum(Ns), r)).astype(np.float32)
    import lora_linear_layer_amd as lla
    got = run_group(g, r, 16.0, flags=lla.LORA_FLAG_ACCUM_GRADS, grads_init=(dA0, dB0))
    _, dAs, dBs = oracle.group_backward(hv["dY"], hv["X"], hv["W"], hv["A"], hv["B"], 0.5)
    a0 = host_view({"X": dA0}, "bf16")["X"]
    b0 = host_view({"X": dB0}, "bf16")["X"]
    assert rel_err(np.vstack(got["dA"]), np.vstack(dAs) + a0) <= DIAG
    assert rel_err(np.vstack(got["dB"]), np.vstack(dBs) + b0) <= DIAG


@pytest.mark.parametrize("r", [8, 24])
def test_one_member_group_is_the_plain_layer(r):
    """A group of one member runs the plain layer's kernels (r = 8: U and V
    formed in the GEMM tiles): every output bit-identical to lora_linear_*."""
    M, K, N = 300, 264, 520
    g = group_inputs(M, K, (N,), r, seed=77)
    got = run_group(g, r, 32.0)
    inp = {"X": g["X"], "W": g["W"][0], "A": g["A"][0], "B": g["B"][0], "dY": g["dY"][0]}
    plain = run_linear(inp, r, 32.0, "bf16")
    for k in ("H", "U", "dA", "dB"):
        np.testing.assert_array_equal(got[k][0].view(np.uint32), plain[k].view(np.uint32), err_msg=k)
    np.testing.assert_array_equal(got["dX"].view(np.uint32), plain["dX"].view(np.uint32), err_msg="dX")


def test_group_rejects_unsupported():
    import lora_linear_layer_amd as lla
    with pytest.raises(lla.LoraError, match="exceeds 192"):
        lla.lora_group_workspace_size(lla.GroupDesc(64, 256, (256, 256), 100, 16.0))
    with pytest.raises(lla.LoraError, match="multiple of 8"):
        lla.lora_group_workspace_size(lla.GroupDesc(64, 256, (256, 12), 8, 16.0))
    with pytest.raises(lla.LoraError, match="bf16"):
        lla.lora_group_workspace_size(lla.GroupDesc(64, 256, (256,), 8, 16.0, lla.LORA_DTYPE_F32))
