"""The allocation-free backward (lora_linear_bwd_noalloc) against the
workspace backward (lora_linear_bwd) and the oracle.

Two calls in a row share the library's static device array: first a larger
problem whose backward uses every region of it (streamed V pass with
contraction chunks, split-M partials of both adapter gradients, rank planes),
then a smaller one (V formed inside the input-gradient GEMM).  Each must give
bitwise the outputs of the workspace entry point on the same inputs, and the
oracle's within the bound of the float32 accumulation plus one bf16 rounding.
A descriptor whose backward needs more than the array holds is refused before
anything is enqueued.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import device_inputs, host_view, rel_err, to_np

pytestmark = pytest.mark.gpu

DIAG = 4e-3


def backward_both(lla, sh, dd, U):
    """(noalloc outputs, workspace outputs) for one set of device inputs."""
    desc = lla.Desc(sh.M, sh.K, sh.N, sh.r, sh.alpha)
    outs = []
    for noalloc in (True, False):
        dX = torch.full((sh.M, sh.K), float("nan"), dtype=torch.bfloat16, device="cuda")
        dA = torch.full((sh.r, sh.K), float("nan"), dtype=torch.bfloat16, device="cuda")
        dB = torch.full((sh.N, sh.r), float("nan"), dtype=torch.bfloat16, device="cuda")
        if noalloc:
            lla.lora_linear_bwd_noalloc(desc, dd["dY"], dd["X"], dd["W"], dd["A"], dd["B"], U, dX, dA, dB)
        else:
            ws = torch.full((lla.lora_linear_workspace_size(desc),), 0xFF, dtype=torch.uint8, device="cuda")
            lla.lora_linear_bwd(desc, dd["dY"], dd["X"], dd["W"], dd["A"], dd["B"], U, dX, dA, dB, ws=ws)
        torch.cuda.synchronize()
        outs.append({"dX": to_np(dX), "dA": to_np(dA), "dB": to_np(dB)})
    return outs


@pytest.mark.parametrize("save_u", [True, False])
def test_noalloc_backward_matches_workspace_backward(save_u):
    import lora_linear_layer_amd as lla
    cases = [workloads.LinearShape("big", 1000, 392, 520, 24, 32.0, 71),     # streamed V, r > 16
             workloads.LinearShape("small", 300, 136, 264, 8, 32.0, 72)]     # V in the dX GEMM
    for sh in cases:
        print(f"noalloc backward {sh.name}: M={sh.M} K={sh.K} N={sh.N} r={sh.r} saved U={save_u}", flush=True)
        inp = workloads.make_linear_inputs(sh)
        dd = device_inputs(inp, "bf16")
        U = None
        if save_u:
            U = torch.empty((sh.M, sh.r), dtype=torch.float32, device="cuda")
            H = torch.empty((sh.M, sh.N), dtype=torch.bfloat16, device="cuda")
            lla.lora_linear_fwd(lla.Desc(sh.M, sh.K, sh.N, sh.r, sh.alpha), dd["X"], dd["W"], dd["A"], dd["B"], H, U)
        got, ref_ws = backward_both(lla, sh, dd, U)
        for k in got:
            np.testing.assert_array_equal(got[k].view(np.uint32), ref_ws[k].view(np.uint32),
                                          err_msg=f"{sh.name} {k}: noalloc differs from the workspace entry point")
        hv = host_view(inp, "bf16")
        dX, dA, dB = oracle.backward(hv["dY"], hv["X"], hv["W"], hv["A"], hv["B"], sh.scale)
        errs = {"dX": rel_err(got["dX"], dX), "dA": rel_err(got["dA"], dA), "dB": rel_err(got["dB"], dB)}
        print(f"  errors {errs}", flush=True)
        assert all(e <= DIAG for e in errs.values()), errs


def test_noalloc_refuses_what_does_not_fit():
    import lora_linear_layer_amd as lla
    # 2^20 tokens at r = 64: V and U alone are 512 MB
    desc = lla.Desc(1 << 20, 64, 64, 64, 16.0)
    with pytest.raises(lla.LoraError, match="allocation-free"):
        lla.lora_linear_bwd_noalloc(desc, 16, 32, 48, 64, 80, None, None, 96, 112)
