"""GPU parity of lora_merge (W_out = W + sign * s * B A) against the oracle's
merged weight, through the C ABI.

Graded bound as for the layer outputs (max|err| / max|ref| <= 1e-2 bf16,
1e-5 float32, the oracle on the float32 draws); diagnostic bound on exactly the
values the GPU received: every element within one bf16 rounding (2^-8 of its
magnitude) plus float32 accumulation error.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import BF16_TOL, F32_TOL, DTYPES, host_view, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = {"bf16": BF16_TOL, "f32": F32_TOL}


def merge_inputs(N, K, r, seed):
    sh = workloads.LinearShape("merge", 8, K, N, r, 32.0, seed)
    inp = workloads.make_linear_inputs(sh)
    return sh, {"W": inp["W"], "A": inp["A"], "B": inp["B"]}


def gpu_merge(inp, sh, dtype, sign=1, in_place=False):
    import lora_linear_layer_amd as lla
    tdt = DTYPES[dtype]
    W, A, B = (to_dev(inp[k], tdt) for k in ("W", "A", "B"))
    desc = lla.Desc(1, sh.K, sh.N, sh.r, sh.alpha, lla.LORA_DTYPE_BF16 if dtype == "bf16" else lla.LORA_DTYPE_F32)
    out = W if in_place else torch.empty_like(W)
    lla.lora_merge(desc, W, A, B, out, sign)
    torch.cuda.synchronize()
    return to_np(out)


def check_merge(got, inp, sh, dtype, sign):
    s = sign * sh.scale
    graded = oracle.merged_weight(inp["W"], inp["A"], inp["B"], s)
    assert rel_err(got, graded) <= TOL[dtype]
    hv = host_view(inp, dtype)
    ref = oracle.merged_weight(hv["W"], hv["A"], hv["B"], s)
    bound = (2.0 ** -8 if dtype == "bf16" else 1e-6) * np.abs(ref) + 1e-6 * np.abs(ref).max()
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{bad.sum()} elements outside one rounding, worst {np.abs(got - ref).max()}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,K,r", [(264, 392, 8), (33, 8, 1), (1000, 136, 100), (64, 4104, 128),
                                   (4096, 4096, 8), (14336, 4096, 64),
                                   # bf16 ranks r >= 16 take the MFMA form (B rows unaligned when r % 8 != 0):
                                   # every rank padding (32, 64, 96, 128) with ragged rows and columns
                                   (520, 264, 16), (1030, 96, 24), (200, 392, 32), (130, 72, 40),
                                   (4100, 520, 96), (77, 8, 120), (300, 136, 17), (260, 200, 60)])
@pytest.mark.parametrize("sign", [1, -1])
def test_merge_parity(N, K, r, sign, dtype):
    sh, inp = merge_inputs(N, K, r, N + K + r)
    print(f"merge N={N} K={K} r={r} sign={sign} {dtype}", flush=True)
    check_merge(gpu_merge(inp, sh, dtype, sign), inp, sh, dtype, sign)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_in_place_equals_out_of_place(dtype):
    sh, inp = merge_inputs(520, 264, 16, 3)
    a = gpu_merge(inp, sh, dtype, in_place=False)
    b = gpu_merge(inp, sh, dtype, in_place=True)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_then_unmerge_restores_w(dtype):
    import lora_linear_layer_amd as lla
    sh, inp = merge_inputs(300, 512, 8, 4)
    tdt = DTYPES[dtype]
    W, A, B = (to_dev(inp[k], tdt) for k in ("W", "A", "B"))
    W0 = to_np(W)
    desc = lla.Desc(1, sh.K, sh.N, sh.r, sh.alpha, lla.LORA_DTYPE_BF16 if dtype == "bf16" else lla.LORA_DTYPE_F32)
    lla.lora_merge(desc, W, A, B, W, 1)
    lla.lora_merge(desc, W, A, B, W, -1)
    torch.cuda.synchronize()
    # two roundings to the dtype: the merged value's (at most half a unit of
    # it, carried through) and the restored value's (half a unit of W)
    hv = host_view(inp, dtype)
    Wm = oracle.merged_weight(hv["W"], hv["A"], hv["B"], sh.scale)
    unit = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    tol = unit * (np.abs(W0) + np.abs(Wm)) + 1e-6 * np.abs(W0).max()
    assert np.all(np.abs(to_np(W) - W0) <= tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_zero_b_is_exact(dtype):
    sh, inp = merge_inputs(96, 200, 8, 5)
    inp = dict(inp, B=np.zeros_like(inp["B"]))
    got = gpu_merge(inp, sh, dtype)
    np.testing.assert_array_equal(got.view(np.uint32), host_view(inp, dtype)["W"].astype(np.float32).view(np.uint32))
