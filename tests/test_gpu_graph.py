"""HIP graph capture of a forward + backward step through the C ABI.

The library's host side only launches kernels on the caller's stream, so a
step can be recorded into a graph and replayed.  Each replay here follows
eager work on the same buffers (outputs overwritten with NaN, the workspace
with 0xFF bytes, a forward + backward of other inputs with the same
workspace) and a synchronisation, and must reproduce the eager results bit
for bit.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_harness import device_inputs, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("r", [8, 64])
def test_graph_replay_matches_eager(r):
    import lora_linear_layer_amd as lla
    sh = workloads.LinearShape("case", 520, 392, 264, r, 32.0, 11)
    other = workloads.LinearShape("case", 520, 392, 264, r, 32.0, 12)
    dd = device_inputs(workloads.make_linear_inputs(sh), "bf16")
    d2 = device_inputs(workloads.make_linear_inputs(other), "bf16")
    desc = lla.Desc(sh.M, sh.K, sh.N, r, sh.alpha)
    ws = torch.empty(lla.lora_linear_workspace_size(desc), dtype=torch.uint8, device="cuda")
    bf = torch.bfloat16

    def buffers():
        return {"H": torch.empty((sh.M, sh.N), dtype=bf, device="cuda"),
                "U": torch.empty((sh.M, r), dtype=torch.float32, device="cuda"),
                "dX": torch.empty((sh.M, sh.K), dtype=bf, device="cuda"),
                "dA": torch.empty((r, sh.K), dtype=bf, device="cuda"),
                "dB": torch.empty((sh.N, r), dtype=bf, device="cuda")}

    def step(d, o):
        lla.lora_linear_fwd(desc, d["X"], d["W"], d["A"], d["B"], o["H"], o["U"], ws=ws)
        lla.lora_linear_bwd(desc, d["dY"], d["X"], d["W"], d["A"], d["B"], o["U"], o["dX"], o["dA"], o["dB"], ws=ws)

    out, scratch_out = buffers(), buffers()
    step(dd, out)
    torch.cuda.synchronize()
    eager = {k: to_np(v) for k, v in out.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(dd, out)
    torch.cuda.synchronize()
    for rep in range(3):
        for v in out.values():
            v.fill_(float("nan"))
        ws.fill_(0xFF)
        step(d2, scratch_out)          # eager work on the same workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            np.testing.assert_array_equal(to_np(v).view(np.uint32), eager[k].view(np.uint32),
                                          err_msg=f"replay {rep}: {k}")
