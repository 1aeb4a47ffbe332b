"""The auto-tuner on the GPU: lora_tune_linear probes the launch parameters of
a layer shape, caches the fastest, and the entry points then use them.
Whatever it picks, the outputs still match the oracle (the candidates differ
only in how the contractions are split and chunked), and the cache survives a
save / clear / load round trip.  The cache is cleared afterwards so that the
other tests run with the built-in rules.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import device_inputs, host_view, rel_err, run_linear, to_np

pytestmark = pytest.mark.gpu

DIAG = 4e-3


def buffers(lla, sh, dd, quant):
    M, K, N, r = sh.M, sh.K, sh.N, sh.r
    bf = torch.bfloat16
    return dict(H=torch.empty((M, N), dtype=bf, device="cuda"), U=torch.empty((M, r), dtype=torch.float32, device="cuda"),
                dX=torch.empty((M, K), dtype=bf, device="cuda"), dA=torch.empty((r, K), dtype=bf, device="cuda"),
                dB=torch.empty((N, r), dtype=bf, device="cuda"))


@pytest.mark.parametrize("quant", [False, True])
def test_tune_then_use(quant, tmp_path):
    import lora_linear_layer_amd as lla
    # few output tiles (a split contraction is a real choice) and r = 24 (streamed U, V passes)
    sh = workloads.LinearShape("t", 1024, 2048, 1536, 24, 32.0, 91, quant)
    inp = workloads.make_qlora_inputs(sh) if quant else workloads.make_linear_inputs(sh)
    dd = device_inputs(inp, "bf16", quant=quant)
    desc = lla.Desc(sh.M, sh.K, sh.N, sh.r, sh.alpha)
    b = buffers(lla, sh, dd, quant)
    wargs = dict(Wq=dd["codes"], absmax=dd["absmax"], codebook=dd["codebook"]) if quant else dict(W=dd["W"])
    lla.lora_tuner_clear()
    try:
        chosen = lla.lora_tune_linear(desc, dd["X"], dd["A"], dd["B"], b["H"], b["U"], dd["dY"], b["dX"], b["dA"],
                                      b["dB"], reps=3, **wargs)
        print(f"tuned (4-bit={quant}): {chosen}", flush=True)
        assert chosen["fwd_us"] <= chosen["default_fwd_us"] and chosen["bwd_us"] <= chosen["default_bwd_us"]
        found = lla.lora_tuner_lookup(desc, quant)
        assert found == {k: chosen[k] for k in found}
        # the entry points now run with the tuned parameters: still the oracle's results
        got = run_linear(inp, sh.r, sh.alpha, "bf16", quant=quant)
        ref_in = dict(host_view(inp, "bf16"))
        if quant:
            ref_in["W"] = oracle.dequant4(inp["codes"], inp["absmax"], oracle.codebook4(), out="bf16")
        H, U = oracle.forward(ref_in["X"], ref_in["W"], ref_in["A"], ref_in["B"], sh.scale)
        dX, dA, dB = oracle.backward(ref_in["dY"], ref_in["X"], ref_in["W"], ref_in["A"], ref_in["B"], sh.scale)
        errs = {k: rel_err(got[k], v) for k, v in (("H", H), ("U", U), ("dX", dX), ("dA", dA), ("dB", dB))}
        print(f"  errors with the tuned parameters {errs}", flush=True)
        assert all(e <= DIAG for e in errs.values()), errs
        # save, clear, load
        path = tmp_path / "tune.txt"
        lla.lora_tuner_save(path)
        lla.lora_tuner_clear()
        assert lla.lora_tuner_lookup(desc, quant) is None
        lla.lora_tuner_load(path)
        assert lla.lora_tuner_lookup(desc, quant) == found
    finally:
        lla.lora_tuner_clear()
