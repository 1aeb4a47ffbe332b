"""The torch.autograd wrappers (lora_linear_layer_amd.layer) on the GPU: forward
and backward through autograd, with leading batch dimensions, against the
oracle on exactly the values the GPU received (diagnostic bound: one bf16
rounding of each output, or 1e-5 in float32), and the merged weight of the
module against the layer's own forward."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import F32_TOL, DTYPES, host_view, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

DIAG = {"bf16": 4e-3, "f32": F32_TOL}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lora_linear_module_autograd(dtype):
    from lora_linear_layer_amd.layer import LoraLinear
    sh = workloads.LinearShape("layer", 80, 264, 136, 8, 32.0, 21)
    inp = workloads.make_linear_inputs(sh)
    tdt = DTYPES[dtype]
    layer = LoraLinear(sh.K, sh.N, sh.r, sh.alpha, weight=to_dev(inp["W"], tdt), dtype=tdt, device="cuda")
    with torch.no_grad():
        layer.lora_A.copy_(to_dev(inp["A"], tdt))
        layer.lora_B.copy_(to_dev(inp["B"], tdt))
    x = to_dev(inp["X"], tdt).reshape(2, 40, sh.K).requires_grad_(True)
    dY = to_dev(inp["dY"], tdt).reshape(2, 40, sh.N)
    y = layer(x)
    y.backward(dY)
    torch.cuda.synchronize()
    assert layer.weight.grad is None
    hv = host_view(inp, dtype)
    H, _ = oracle.forward(hv["X"], hv["W"], hv["A"], hv["B"], sh.scale)
    dX, dA, dB = oracle.backward(hv["dY"], hv["X"], hv["W"], hv["A"], hv["B"], sh.scale)
    got = {"H": to_np(y).reshape(sh.M, sh.N), "dX": to_np(x.grad).reshape(sh.M, sh.K),
           "dA": to_np(layer.lora_A.grad), "dB": to_np(layer.lora_B.grad)}
    for k, ref in (("H", H), ("dX", dX), ("dA", dA), ("dB", dB)):
        assert rel_err(got[k], ref) <= DIAG[dtype], (k, rel_err(got[k], ref))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qlora_function_autograd(dtype):
    from lora_linear_layer_amd.layer import QLoraLinearFunction
    sh = workloads.LinearShape("qlayer", 64, 256, 264, 16, 32.0, 22, True)
    inp = workloads.make_qlora_inputs(sh)
    tdt = DTYPES[dtype]
    codes = torch.from_numpy(inp["codes"]).cuda()
    absmax = torch.from_numpy(np.ascontiguousarray(inp["absmax"]).view(np.int16)).cuda()
    cb = torch.from_numpy(inp["codebook"]).cuda()
    A = to_dev(inp["A"], tdt).requires_grad_(True)
    B = to_dev(inp["B"], tdt).requires_grad_(True)
    x = to_dev(inp["X"], tdt).requires_grad_(True)
    y = QLoraLinearFunction.apply(x, codes, absmax, cb, A, B, sh.alpha)
    y.backward(to_dev(inp["dY"], tdt))
    torch.cuda.synchronize()
    hv = host_view(inp, dtype)
    W = oracle.dequant4(inp["codes"], inp["absmax"], oracle.codebook4(), out="bf16" if dtype == "bf16" else "f32")
    H, _ = oracle.forward(hv["X"], W, hv["A"], hv["B"], sh.scale)
    dX, dA, dB = oracle.backward(hv["dY"], hv["X"], W, hv["A"], hv["B"], sh.scale)
    for k, g, ref in (("H", y, H), ("dX", x.grad, dX), ("dA", A.grad, dA), ("dB", B.grad, dB)):
        assert rel_err(to_np(g), ref) <= DIAG[dtype], (k, rel_err(to_np(g), ref))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_module_merged_weight_reproduces_forward(dtype):
    """x W'^T with the merged weight W' = W + s B A equals the layer's forward
    (the two differ only by roundings), and unmerging restores W."""
    from lora_linear_layer_amd.layer import LoraLinear
    sh = workloads.LinearShape("merge", 96, 512, 264, 16, 32.0, 23)
    inp = workloads.make_linear_inputs(sh)
    tdt = DTYPES[dtype]
    layer = LoraLinear(sh.K, sh.N, sh.r, sh.alpha, weight=to_dev(inp["W"], tdt), dtype=tdt, device="cuda")
    with torch.no_grad():
        layer.lora_A.copy_(to_dev(inp["A"], tdt))
        layer.lora_B.copy_(to_dev(inp["B"], tdt))
        x = to_dev(inp["X"], tdt)
        y = layer(x)
        Wm = layer.merged_weight()
        y_merged = x.float() @ Wm.float().t().contiguous()
    torch.cuda.synchronize()
    hv = host_view(inp, dtype)
    ref = oracle.merged_weight(hv["W"], hv["A"], hv["B"], sh.scale)
    assert rel_err(to_np(Wm), ref) <= DIAG[dtype]
    # merged weight rounded to the dtype: the products differ by that rounding
    assert rel_err(to_np(y_merged), to_np(y).astype(np.float64)) <= (2e-2 if dtype == "bf16" else 1e-5)
    with torch.no_grad():
        layer.weight.copy_(Wm)
        restored = layer.merged_weight(-1)
    assert rel_err(to_np(restored), hv["W"]) <= (2 ** -7 if dtype == "bf16" else 1e-6)


def test_module_with_transposed_weight_is_bit_identical():
    """LoraLinear(keep_transposed_weight=True): the backward reads the module's
    W^T buffer; outputs and gradients bit-identical to the module without it,
    also after the weight changes and refresh_transposed_weight()."""
    from lora_linear_layer_amd.layer import LoraLinear
    sh = workloads.LinearShape("layer_wt", 300, 520, 264, 16, 32.0, 23)
    inp = workloads.make_linear_inputs(sh)
    bf = torch.bfloat16
    mods = [LoraLinear(sh.K, sh.N, sh.r, sh.alpha, weight=to_dev(inp["W"], bf), device="cuda",
                       keep_transposed_weight=k) for k in (False, True)]
    for m in mods:
        with torch.no_grad():
            m.lora_A.copy_(to_dev(inp["A"], bf))
            m.lora_B.copy_(to_dev(inp["B"], bf))
    assert mods[1].weight_t.shape == (sh.K, sh.N)
    for step in range(2):
        res = []
        for m in mods:
            m.zero_grad(set_to_none=True)
            x = to_dev(inp["X"], bf).requires_grad_(True)
            y = m(x)
            y.backward(to_dev(inp["dY"], bf))
            res.append([y, x.grad, m.lora_A.grad, m.lora_B.grad])
        torch.cuda.synchronize()
        for name, a, b in zip(("H", "dX", "dA", "dB"), *res):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"step {step}: {name}"
        with torch.no_grad():                      # a new frozen weight for the second round
            for m in mods:
                m.weight.mul_(0.5)
            mods[1].refresh_transposed_weight()
