"""The decoder-layer workload exactly as bench.py runs it, against the oracle.

Seven LoRA linears (q, k, v, o, gate, up, down; M = 4096, r = 64, alpha = 16)
go through bench.py's own runner: q/k/v read one X and gate/up read one X
(bench.share_inputs), every call shares one workspace sized for the largest
of the seven descriptors (bench.Stepper), the backward reading W^T
(bench.add_wt, the default layout), the forwards run in order and the
backwards in reverse.  Every element of every output of every linear is
compared with the float64 oracle on the float32 draws (the graded bound), and
a second step on the same workspace must reproduce the first bit for bit.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import workloads
from gpu_harness import BF16_TOL, device_inputs, rel_err, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

OUTPUTS = ("H", "U", "dX", "dA", "dB")


def test_decoder_layer_as_benched():
    import lora_linear_layer_amd as lla
    wl = workloads.workload("decoder_layer_r64")
    dev = torch.device("cuda:0")
    inps = [workloads.make_linear_inputs(sh) for sh in wl.linears]
    bench.share_inputs(wl, inps)                     # the host copies share X the same way
    layer = [device_inputs(inp, "bf16") for inp in inps]
    bench.share_inputs(wl, layer)
    assert layer[1]["X"] is layer[0]["X"] and layer[5]["X"] is layer[4]["X"]
    bench.add_outputs(lla, torch, wl, layer, dev)
    bench.add_wt(lla, torch, wl, layer)               # the backward reads W^T, as bench.py does by default
    stepper = bench.Stepper(lla, torch, [layer], dev)
    assert stepper.ws_bytes == max(lla.lora_linear_workspace_size(d["desc"]) for d in layer)
    print(f"decoder layer, one workspace of {stepper.ws_bytes} bytes", flush=True)
    runs = []
    for _ in range(2):
        stepper.step(layer)
        torch.cuda.synchronize()
        runs.append([{k: to_np(d[k]) for k in OUTPUTS} for d in layer])
    for li, sh in enumerate(wl.linears):
        for k in OUTPUTS:
            np.testing.assert_array_equal(runs[0][li][k].view(np.uint32), runs[1][li][k].view(np.uint32),
                                          err_msg=f"{sh.name} {k}: second step differs")
    for sh, inp, got in zip(wl.linears, inps, runs[1]):
        X, W, A, B, dY, s = inp["X"], inp["W"], inp["A"], inp["B"], inp["dY"], sh.scale
        H, U = oracle.forward(X, W, A, B, s)
        dX, dA, dB = oracle.backward(dY, X, W, A, B, s)
        errs = {k: rel_err(got[k], ref) for k, ref in (("H", H), ("U", U), ("dX", dX), ("dA", dA), ("dB", dB))}
        print(f"  {sh.name}: graded errors {errs}", flush=True)
        bad = {k: e for k, e in errs.items() if not e <= BF16_TOL}
        assert not bad, f"{sh.name}: {errs} exceed {BF16_TOL}"


def test_decoder_layer_grouped_as_benched():
    """The same layer as bench.py --grouped runs it: q/k/v one grouped call and
    gate/up one grouped call (stacked operands, one pass over X for all their
    U, dX of the shared input summed over the members), o and down alone.
    Every member's H, U, dA, dB and every call's dX against the oracle
    (group_forward / group_backward for the groups), graded bound."""
    import lora_linear_layer_amd as lla
    wl = workloads.workload("decoder_layer_r64")
    dev = torch.device("cuda:0")
    inps = [workloads.make_linear_inputs(sh) for sh in wl.linears]
    bench.share_inputs(wl, inps)
    layer = [device_inputs(inp, "bf16") for inp in inps]
    bench.share_inputs(wl, layer)
    bench.add_outputs(lla, torch, wl, layer, dev)
    bench.add_wt(lla, torch, wl, layer)
    units = bench.step_units(wl, True)
    glayer = bench.group_layer(lla, torch, wl, layer, units, dev)
    stepper = bench.Stepper(lla, torch, [glayer], dev)
    print(f"grouped decoder layer: calls {[u.name for u in units]}, workspace {stepper.ws_bytes} bytes", flush=True)
    stepper.step(glayer)
    torch.cuda.synchronize()
    for u, d in zip(units, glayer):
        got = {k: to_np(d[k]) for k in OUTPUTS}
        mem = [wl.linears[i] for i in u.members]
        mi = [inps[i] for i in u.members]
        s = mem[0].scale
        X = mi[0]["X"]
        outs = oracle.group_forward(X, [m["W"] for m in mi], [m["A"] for m in mi], [m["B"] for m in mi], s)
        dX, dAs, dBs = oracle.group_backward([m["dY"] for m in mi], X, [m["W"] for m in mi],
                                             [m["A"] for m in mi], [m["B"] for m in mi], s)
        errs = {"dX": rel_err(got["dX"], dX)}
        n0, r = 0, u.r
        for k, (sh, (H, U), dA, dB) in enumerate(zip(mem, outs, dAs, dBs)):
            errs[f"{sh.name} H"] = rel_err(got["H"][:, n0:n0 + sh.N], H)
            errs[f"{sh.name} U"] = rel_err(got["U"][:, k * r:(k + 1) * r], U)
            errs[f"{sh.name} dA"] = rel_err(got["dA"][k * r:(k + 1) * r], dA)
            errs[f"{sh.name} dB"] = rel_err(got["dB"][n0:n0 + sh.N], dB)
            n0 += sh.N
        print(f"  {u.name}: graded errors {errs}", flush=True)
        bad = {k: e for k, e in errs.items() if not e <= BF16_TOL}
        assert not bad, f"{u.name}: {bad} exceed {BF16_TOL}"


def test_decoder_layer_grouped_norm_as_benched():
    """bench.py --grouped --norm: q/k/v and gate/up as grouped calls behind an
    RMSNorm each (W folded with g in place, the layer reading the raw X), o and
    down plain.  Members against oracle.norm_forward / norm_backward with the
    host copy of g; a group's dX against the sum of its members' input
    gradients; graded bound."""
    import lora_linear_layer_amd as lla
    wl = workloads.workload("decoder_layer_r64")
    dev = torch.device("cuda:0")
    inps = [workloads.make_linear_inputs(sh) for sh in wl.linears]
    bench.share_inputs(wl, inps)
    layer = [device_inputs(inp, "bf16") for inp in inps]
    bench.share_inputs(wl, layer)
    bench.add_outputs(lla, torch, wl, layer, dev)
    bench.add_norm(lla, torch, wl, layer, dev, seed=7000)
    bench.add_wt(lla, torch, wl, layer)
    units = bench.step_units(wl, True)
    glayer = bench.group_layer(lla, torch, wl, layer, units, dev)
    stepper = bench.Stepper(lla, torch, [glayer], dev)
    print(f"grouped decoder layer with RMSNorm: calls {[u.name for u in units]}", flush=True)
    stepper.step(glayer)
    torch.cuda.synchronize()
    eps = bench.NORM_EPS
    for u, d in zip(units, glayer):
        got = {k: to_np(d[k]) for k in OUTPUTS}
        mem = [wl.linears[i] for i in u.members]
        mi = [inps[i] for i in u.members]
        s = mem[0].scale
        X = mi[0]["X"]
        errs = {}
        if "g" in d:
            g = to_np(d["g"])
            dX = 0.0
            n0 = 0
            for k, (sh, m) in enumerate(zip(mem, mi)):
                H, U, _ = oracle.norm_forward(X, g, eps, m["W"], m["A"], m["B"], s)
                dXk, dA, dB = oracle.norm_backward(m["dY"], X, g, eps, m["W"], m["A"], m["B"], s)
                dX = dX + dXk
                errs[f"{sh.name} H"] = rel_err(got["H"][:, n0:n0 + sh.N], H)
                errs[f"{sh.name} U"] = rel_err(got["U"][:, k * u.r:(k + 1) * u.r], U)
                errs[f"{sh.name} dA"] = rel_err(got["dA"][k * u.r:(k + 1) * u.r], dA)
                errs[f"{sh.name} dB"] = rel_err(got["dB"][n0:n0 + sh.N], dB)
                n0 += sh.N
            errs["dX"] = rel_err(got["dX"], dX)
        else:
            m = mi[0]
            H, U = oracle.forward(X, m["W"], m["A"], m["B"], s)
            dX, dA, dB = oracle.backward(m["dY"], X, m["W"], m["A"], m["B"], s)
            errs = {k: rel_err(got[k], ref) for k, ref in (("H", H), ("U", U), ("dX", dX), ("dA", dA), ("dB", dB))}
        print(f"  {u.name}: graded errors {errs}", flush=True)
        bad = {k: e for k, e in errs.items() if not e <= BF16_TOL}
        assert not bad, f"{u.name}: {bad} exceed {BF16_TOL}"
