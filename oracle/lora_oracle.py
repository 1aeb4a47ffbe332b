"""Plain float64 CPU oracle for the LoRA linear layer -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the HIP library or its Python
binding, and the product path never calls it.

Everything here is the textbook definition written out in numpy float64 on
the inputs as given (promoted exactly to float64).  The d x d product B.A is
never formed except in `merged_weight`, which exists for the deployment
identity and for tests on tiny shapes.

Sources (the four web pages about Unsloth; page titles as printed):
  [P1] "UnSloth加速库集成：编译级优化带来的性能飞跃" (UnSloth integration:
       compile-level optimisation), section "为什么标准LoRA会慢？" (why
       standard LoRA is slow): dW = B A with A in R^{r x d}, B in R^{d x r},
       forward h = W x + B (A x).
  [P3] "Unsloth — 微调 2-5x 加速", section "核心要点" (core points), item 2:
       the backward products are re-associated so that only rank-r
       intermediates exist; item 3: 4-bit weights are dequantised inside the
       matmul.
  [P4] "ms-swift高效微调组合：LoRA+UnSloth提速实践", section 1.2 "梯度计算
       绕过Autograd": LoRA gradients written in closed form (the printed
       formulas drop the input and the scale; the forms below are the exact
       vector-Jacobian products of the forward).
  [P2] "ms-swift框架下UnSloth与Liger-Kernel优化实战", section "UnSloth：让
       LoRA真正“低秩”起来": the backbone W is frozen, so no dW exists.

Readings where the pages are silent or garbled:
  * scale s = lora_alpha / r multiplies the low-rank term (the pages show
    lora_alpha as a config knob but no formula);
  * one token per row: X[M,K] holds tokens x d_in, W[N,K] is d_out x d_in,
    A[r,K], B[N,r]; H = X W^T + s (X A^T) B^T is P1's h = W x + B(A x) with
    x a column of X^T;
  * no bias, no dropout.
"""
from __future__ import annotations

from statistics import NormalDist

import numpy as np

__all__ = [
    "lora_scale", "forward", "backward", "backward_dx", "backward_lora",
    "merged_weight", "group_forward", "group_backward", "rms_norm", "norm_forward", "norm_backward",
    "bf16_round", "f16_to_f64", "codebook4", "dequant4",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def lora_scale(alpha: float, r: int) -> float:
    """s = lora_alpha / r."""
    return float(alpha) / float(r)


def forward(X, W, A, B, s):
    """[P1] forward, row form: U = X A^T, H = X W^T + s U B^T.

    Returns (H, U) in float64.
    """
    X, W, A, B = _f64(X), _f64(W), _f64(A), _f64(B)
    U = X @ A.T
    H = X @ W.T + float(s) * (U @ B.T)
    return H, U


def backward_dx(dY, W, A, B, s):
    """Input gradient of L = <dY, H>: dX = dY W + s (dY B) A  ([P3] item 2 order).

    Row-local: rows of dX depend only on the same rows of dY.
    """
    dY, W, A, B = _f64(dY), _f64(W), _f64(A), _f64(B)
    V = dY @ B
    return dY @ W + float(s) * (V @ A)


def backward_lora(dY, X, A, B, s):
    """Adapter gradients of L = <dY, H>  ([P4] section 1.2, corrected).

    dA = s (dY B)^T X  [r,K];  dB = s dY^T (X A^T)  [N,r].  Both sum over tokens.
    """
    dY, X, A, B = _f64(dY), _f64(X), _f64(A), _f64(B)
    V = dY @ B
    U = X @ A.T
    dA = float(s) * (V.T @ X)
    dB = float(s) * (dY.T @ U)
    return dA, dB


def backward(dY, X, W, A, B, s):
    """(dX, dA, dB); W is frozen so no dW is produced ([P2])."""
    dX = backward_dx(dY, W, A, B, s)
    dA, dB = backward_lora(dY, X, A, B, s)
    return dX, dA, dB


def merged_weight(W, A, B, s):
    """W' = W + s B A: the adapter folded into the frozen weight before
    deployment ([P2] section "设计权衡与最佳实践", item 4, merge-and-unload
    for inference engines); with -s it removes the adapter again (unmerge).
    Forms the N x K product B A, so only for test shapes."""
    return _f64(W) + float(s) * (_f64(B) @ _f64(A))


# ----------------------------------------------------------------------------
# Linears that read the same input
# ----------------------------------------------------------------------------

def group_forward(X, Ws, As, Bs, s):
    """Several LoRA linears applied to one input X (the attention projections
    q, k, v, or the MLP's gate and up: [P4] section 1.2, the fused q_proj
    example, and section 2.3, LoRA on all linear layers).  Each member i is
    its own layer: H_i = X W_i^T + s (X A_i^T) B_i^T.  Returns [(H_i, U_i)]."""
    return [forward(X, W, A, B, s) for W, A, B in zip(Ws, As, Bs)]


def group_backward(dYs, X, Ws, As, Bs, s):
    """Vector-Jacobian products of L = sum_i <dY_i, H_i> for group_forward.
    X feeds every member, so its gradient is the sum of the members' input
    gradients; each member keeps its own dA_i, dB_i.  Returns (dX, [dA_i], [dB_i])."""
    dX = None
    dAs, dBs = [], []
    for dY, W, A, B in zip(dYs, Ws, As, Bs):
        dXi, dAi, dBi = backward(dY, X, W, A, B, s)
        dX = dXi if dX is None else dX + dXi
        dAs.append(dAi)
        dBs.append(dBi)
    return dX, dAs, dBs


# ----------------------------------------------------------------------------
# RMSNorm in front of the layer
# ----------------------------------------------------------------------------

def rms_norm(X, g, eps):
    """RMSNorm over the last axis ([P2] section "关键融合策略解析", RMSNorm +
    Linear: the norm that feeds the attention projections):
    Xn[m, k] = X[m, k] / sqrt(mean_k X[m, k]^2 + eps) * g[k].  Returns (Xn, inv)
    with inv[m] = 1 / sqrt(mean_k X[m, k]^2 + eps)."""
    X, g = _f64(X), _f64(g)
    inv = 1.0 / np.sqrt(np.mean(X * X, axis=1) + float(eps))
    return X * inv[:, None] * g[None, :], inv


def norm_forward(X, g, eps, W, A, B, s):
    """The LoRA linear applied to RMSNorm(X): H = Xn W^T + s (Xn A^T) B^T.
    Returns (H, U, inv) with U = Xn A^T."""
    Xn, inv = rms_norm(X, g, eps)
    H, U = forward(Xn, W, A, B, s)
    return H, U, inv


def norm_backward(dY, X, g, eps, W, A, B, s):
    """Vector-Jacobian products of L = <dY, H> for norm_forward, with respect to
    the raw input X and the adapter (the norm's g is part of the frozen
    backbone, like W: no gradient).  The layer gives dXn = dY W + s (dY B) A and
    dA = s (dY B)^T Xn, dB = s dY^T (Xn A^T); the norm's Jacobian, for one row
    with inv = 1 / sqrt(mean(x^2) + eps), is
        dx = inv * g * dxn - x * inv^3 / K * sum_k g[k] dxn[k] x[k].
    Returns (dX, dA, dB)."""
    X, g = _f64(X), _f64(g)
    Xn, inv = rms_norm(X, g, eps)
    dXn = backward_dx(dY, W, A, B, s)
    dA, dB = backward_lora(dY, Xn, A, B, s)
    K = X.shape[1]
    dot = np.sum(g[None, :] * dXn * X, axis=1)
    dX = inv[:, None] * g[None, :] * dXn - X * (inv ** 3 / K * dot)[:, None]
    return dX, dA, dB


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns float32.

    bfloat16 keeps the top 16 bits of the float32 encoding.  Rounding adds
    0x7FFF plus the lowest kept bit before truncating.  NaN stays NaN.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + keep_lsb) >> 16) << 16
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), f, out)


def f16_to_f64(h) -> np.ndarray:
    """IEEE binary16 bit patterns (or float16 values) to float64, exactly.

    Decoded from the fields: sign, 5-bit exponent (bias 15), 10-bit mantissa.
    """
    bits = np.asarray(h)
    bits = bits.view(np.uint16) if bits.dtype == np.float16 else bits.astype(np.uint16)
    b = bits.astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = (b & 0x3FF).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 1024.0, (e - 15).astype(np.int64))
    sub = sign * np.ldexp(m / 1024.0, -14)
    inf_nan = np.where(m == 0, sign * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 31, inf_nan, normal))


def codebook4() -> np.ndarray:
    """16-entry 4-bit codebook: c_i = Phi^-1((i+0.5)/16) / Phi^-1(15.5/16).

    Evaluated in float64 and rounded once to float32 (returned as float32).
    """
    nd = NormalDist()
    top = nd.inv_cdf(15.5 / 16.0)
    vals = [nd.inv_cdf((i + 0.5) / 16.0) / top for i in range(16)]
    return np.array(vals, dtype=np.float64).astype(np.float32)


def dequant4(codes, absmax, codebook, out: str = "bf16") -> np.ndarray:
    """Dequantise 4-bit codes ([P3] core point 3: int4 weights restored inside the matmul).

    codes[N, K/2] uint8: element k is the low nibble of byte k/2 when k is
    even, the high nibble when k is odd.  absmax[N, K/64]: fp16, one per block
    of 64 consecutive elements along K.  Each weight is the float32 product
    codebook[code] * float32(absmax) (IEEE, round to nearest even), then for
    out="bf16" rounded to bfloat16; out="f32" keeps the float32 product.
    Returns float32 values [N, K].
    """
    codes = np.asarray(codes, dtype=np.uint8)
    N, half = codes.shape
    K = 2 * half
    idx = np.empty((N, K), dtype=np.int64)
    idx[:, 0::2] = codes & 0x0F
    idx[:, 1::2] = codes >> 4
    cb = np.asarray(codebook, dtype=np.float32)
    scale = f16_to_f64(absmax).astype(np.float32)          # exact: fp16 embeds in fp32
    per_elem = np.repeat(scale, K // scale.shape[1], axis=1)
    # float64 product of two float32 values is exact; one rounding to float32 = IEEE fp32 multiply
    prod = (cb[idx].astype(np.float64) * per_elem.astype(np.float64)).astype(np.float32)
    if out == "f32":
        return prod
    if out == "bf16":
        return bf16_round(prod)
    raise ValueError("out must be 'bf16' or 'f32'")
