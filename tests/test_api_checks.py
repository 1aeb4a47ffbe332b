"""Argument checks of the Python binding and the autograd wrappers (no GPU).

Every call here is refused before the library is reached: wrong shapes,
dtypes or devices of tensor arguments raise in Python, so nothing is ever
enqueued (the tensors live on the CPU).
"""
import pytest
import torch

import lora_linear_layer_amd as lla
from lora_linear_layer_amd.layer import LoraLinearFunction, QLoraLinearFunction

M, K, N, r = 64, 256, 128, 8


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def dense_args(**over):
    a = dict(X=t(M, K), W=t(N, K), A=t(r, K), B=t(N, r), H=t(M, N), U_save=t(M, r, dtype=torch.float32))
    a.update(over)
    return a


def call_fwd(**over):
    a = dense_args(**over)
    lla.lora_linear_fwd(lla.Desc(M, K, N, r, 32.0), a["X"], a["W"], a["A"], a["B"], a["H"], a["U_save"])


@pytest.mark.parametrize("name,bad", [("X", t(M, K + 8)), ("W", t(K, N)), ("A", t(K, r)), ("B", t(r, N)),
                                      ("H", t(M, N + 8)), ("U_save", t(M, r + 1, dtype=torch.float32))])
def test_forward_rejects_wrong_shape(name, bad):
    with pytest.raises(ValueError, match=name):
        call_fwd(**{name: bad})


@pytest.mark.parametrize("name,bad", [("X", t(M, K, dtype=torch.float32)), ("W", t(N, K, dtype=torch.float16)),
                                      ("A", t(r, K, dtype=torch.float32)), ("B", t(N, r, dtype=torch.float32)),
                                      ("U_save", t(M, r))])
def test_forward_rejects_wrong_dtype(name, bad):
    with pytest.raises(TypeError, match=name):
        call_fwd(**{name: bad})


def test_forward_rejects_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        call_fwd()


def test_backward_rejects_float32_grads_for_bf16_descriptor():
    """dA of float32 for a bf16 descriptor would have the kernels write 2-byte
    values into a 4-byte buffer (and the float32 mode 4-byte values into a
    2-byte one): refused."""
    a = dense_args()
    with pytest.raises(TypeError, match="dA"):
        lla.lora_linear_bwd(lla.Desc(M, K, N, r, 32.0), t(M, N), a["X"], a["W"], a["A"], a["B"], a["U_save"],
                            t(M, K), t(r, K, dtype=torch.float32), t(N, r))
    with pytest.raises(ValueError, match="dB"):
        lla.lora_linear_bwd(lla.Desc(M, K, N, r, 32.0), t(M, N), a["X"], a["W"], a["A"], a["B"], a["U_save"],
                            t(M, K), t(r, K), t(r, N))


def test_qlinear_rejects_bad_weight_format():
    d = lla.Desc(M, K, N, r, 32.0)
    good = dict(Wq=t(N, K // 2, dtype=torch.uint8), absmax=t(N, K // 64, dtype=torch.int16),
                codebook=t(16, dtype=torch.float32))
    for name, bad, exc in (("Wq", t(N, K, dtype=torch.uint8), ValueError),
                           ("Wq", t(N, K // 2, dtype=torch.int8), TypeError),
                           ("absmax", t(N, K // 32, dtype=torch.int16), ValueError),
                           ("absmax", t(N, K // 64, dtype=torch.float32), TypeError),
                           ("codebook", t(16, dtype=torch.float16), TypeError),
                           ("codebook", t(15, dtype=torch.float32), ValueError)):
        w = dict(good, **{name: bad})
        with pytest.raises(exc, match=name):
            lla.lora_qlinear_fwd(d, t(M, K), w["Wq"], w["absmax"], w["codebook"], t(r, K), t(N, r), t(M, N))


def test_dequant_and_merge_reject_mismatches():
    with pytest.raises(ValueError, match="W_out"):
        lla.lora_dequant4(t(N, K // 2, dtype=torch.uint8), t(N, K // 64, dtype=torch.int16),
                          t(16, dtype=torch.float32), N, K, lla.LORA_DTYPE_BF16, t(N, K + 64))
    with pytest.raises(TypeError, match="W_out"):
        lla.lora_dequant4(t(N, K // 2, dtype=torch.uint8), t(N, K // 64, dtype=torch.int16),
                          t(16, dtype=torch.float32), N, K, lla.LORA_DTYPE_F32, t(N, K))
    with pytest.raises(ValueError, match="A"):
        lla.lora_merge(lla.Desc(1, K, N, r, 32.0), t(N, K), t(r + 1, K), t(N, r), t(N, K))


def test_autograd_function_rejects_mixed_dtypes():
    """float32 activations into bf16 parameters (the autocast case) are refused
    by the Function before any library call; the module converts them."""
    x = t(M, K, dtype=torch.float32)
    with pytest.raises(TypeError, match="W"):
        LoraLinearFunction.apply(x, t(N, K), t(r, K), t(N, r), 32.0)
    with pytest.raises(TypeError, match="A"):
        QLoraLinearFunction.apply(x, t(N, K // 2, dtype=torch.uint8), t(N, K // 64, dtype=torch.int16),
                                  t(16, dtype=torch.float32), t(r, K), t(N, r), 32.0)
