"""The decoder-layer workload exactly as bench.py runs it, against the oracle.

Seven LoRA linears (q, k, v, o, gate, up, down; M = 4096, r = 64, alpha = 16)
go through bench.py's own runner: q/k/v read one X and gate/up read one X
(bench.share_inputs), every call shares one workspace sized for the largest
of the seven descriptors (bench.Stepper), the forwards run in order and the
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
