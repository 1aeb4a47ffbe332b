"""The backward with the frozen weight given as W^T (LORA_FLAG_W_TRANSPOSED).

lora_transpose_weight must be an exact transpose, and every backward output
(dX, dA, dB) must be bit-identical to the same call with W: the input-gradient
GEMM multiplies the same bf16 values in the same order, it only reads its
weight operand from the other layout.  Covered: the in-tile rank product
(r = 8, 16, whole tiles), the precomputed-Z form with a split contraction
(r = 40), a grouped call and the RMSNorm path.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_harness import to_dev, to_np

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("N,K", [(264, 520), (4096, 4096), (8, 8)])
def test_transpose_weight_is_exact(N, K):
    import lora_linear_layer_amd as lla
    rng = np.random.Generator(np.random.PCG64(N + K))
    W = to_dev(rng.standard_normal((N, K), dtype=np.float32), BF)
    Wt = torch.empty((K, N), dtype=BF, device="cuda")
    lla.lora_transpose_weight(W, Wt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(Wt), _bits(W.t().contiguous()))


def _bwd_pair(M, K, N, r, seed, save_u=True):
    """(outputs with W, outputs with W^T) of one forward + two backwards."""
    import lora_linear_layer_amd as lla
    sh = workloads.LinearShape("wt", M, K, N, r, 2.0 * r, seed)
    inp = workloads.make_linear_inputs(sh)
    d = {k: to_dev(inp[k], BF) for k in ("X", "W", "A", "B", "dY")}
    Wt = torch.empty((K, N), dtype=BF, device="cuda")
    lla.lora_transpose_weight(d["W"], Wt)
    outs = []
    for flags, Wb in ((0, d["W"]), (lla.LORA_FLAG_W_TRANSPOSED, Wt)):
        desc = lla.Desc(M, K, N, r, sh.alpha, lla.LORA_DTYPE_BF16, flags)
        H = torch.empty((M, N), dtype=BF, device="cuda")
        U = torch.empty((M, r), dtype=torch.float32, device="cuda")
        dX = torch.empty((M, K), dtype=BF, device="cuda")
        dA = torch.empty((r, K), dtype=BF, device="cuda")
        dB = torch.empty((N, r), dtype=BF, device="cuda")
        lla.lora_linear_fwd(desc, d["X"], d["W"], d["A"], d["B"], H, U)
        lla.lora_linear_bwd(desc, d["dY"], d["X"], Wb, d["A"], d["B"], U if save_u else None, dX, dA, dB)
        outs.append({"H": H, "dX": dX, "dA": dA, "dB": dB})
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("M,K,N,r", [
    (2048, 4096, 520, 8),     # whole tiles (128 of them): V formed in the tile
    (2048, 4096, 264, 16),
    (300, 264, 520, 40),      # few tiles: split contraction, V from the streamed pass
    (513, 1032, 2056, 128),
])
def test_w_transposed_backward_is_bit_identical(M, K, N, r):
    a, b = _bwd_pair(M, K, N, r, seed=M + N + r)
    for k in ("dX", "dA", "dB"):
        np.testing.assert_array_equal(_bits(a[k]), _bits(b[k]), err_msg=k)


def test_w_transposed_full_projection_is_bit_identical():
    a, b = _bwd_pair(4096, 4096, 4096, 8, seed=11, save_u=False)
    for k in ("dX", "dA", "dB"):
        np.testing.assert_array_equal(_bits(a[k]), _bits(b[k]), err_msg=k)


def test_w_transposed_group_and_norm_are_bit_identical():
    import lora_linear_layer_amd as lla
    M, K, Ns, r = 300, 392, (264, 136, 520), 16
    rng = np.random.Generator(np.random.PCG64(5))
    N, R = sum(Ns), len(Ns) * r
    X = to_dev(rng.standard_normal((M, K), dtype=np.float32), BF)
    W = to_dev(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02), BF)
    A = to_dev(rng.standard_normal((R, K), dtype=np.float32) * np.float32(0.05), BF)
    B = to_dev(rng.standard_normal((N, r), dtype=np.float32) * np.float32(0.02), BF)
    dY = to_dev(rng.standard_normal((M, N), dtype=np.float32), BF)
    g = to_dev(1.0 + 0.2 * rng.standard_normal(K, dtype=np.float32), BF)
    Wt = torch.empty((K, N), dtype=BF, device="cuda")
    lla.lora_transpose_weight(W, Wt)
    outs = []
    for flags, Wb in ((0, W), (lla.LORA_FLAG_W_TRANSPOSED, Wt)):
        gd = lla.GroupDesc(M, K, Ns, r, 32.0, flags=flags)
        U = torch.empty((M, R), dtype=torch.float32, device="cuda")
        H = torch.empty((M, N), dtype=BF, device="cuda")
        dX, dA, dB = (torch.empty(s, dtype=BF, device="cuda") for s in ((M, K), (R, K), (N, r)))
        lla.lora_group_fwd(gd, X, W, A, B, H, U)
        lla.lora_group_bwd(gd, dY, X, Wb, A, B, U, dX, dA, dB)
        # the same stacked weights behind an RMSNorm (W_g = W diag(g); its transpose for the flag)
        Wg = torch.empty_like(W)
        lla.lora_fold_norm_weight(W, g, Wg)
        Wgb = Wg
        if flags:
            Wgb = torch.empty((K, N), dtype=BF, device="cuda")
            lla.lora_transpose_weight(Wg, Wgb)
        inv = torch.empty((M,), dtype=torch.float32, device="cuda")
        nX, nA, nB = (torch.empty(s, dtype=BF, device="cuda") for s in ((M, K), (R, K), (N, r)))
        lla.lora_norm_group_fwd(gd, 1e-6, X, g, Wg, A, B, H, U, inv)
        lla.lora_norm_group_bwd(gd, 1e-6, dY, X, g, Wgb, A, B, U, inv, nX, nA, nB)
        outs.append([dX, dA, dB, nX, nA, nB])
    torch.cuda.synchronize()
    for name, a, b in zip(("dX", "dA", "dB", "norm dX", "norm dA", "norm dB"), *outs):
        np.testing.assert_array_equal(_bits(a), _bits(b), err_msg=name)
