"""Seeded synthetic inputs for the LoRA linear layer (shared by tests, bench and smoke).

This module only *draws* inputs: it holds none of the layer's arithmetic (no
product, no gradient, no dequantisation).  Both the HIP path and the CPU
oracle are fed from here, so the two sides see exactly the same numbers.

Shapes follow the pages' workloads:
  * hidden 4096, rank 8 ("q_proj, hidden_size=4096, rank=8": page "ms-swift高效
    微调组合：LoRA+UnSloth提速实践", section 1.2 "算子融合");
  * max_length 2048 (same page, section 2.2, experiment table);
  * MLP shapes 4096 <-> 11008 and a full decoder layer (Qwen/Llama-7B family,
    pages' model choices), rank 16 / 64;
  * 4-bit frozen weights with rank 16, alpha 32 (page "ms-swift框架下UnSloth与
    Liger-Kernel优化实战", code listing with load_in_4bit=True).
The pages measure on a dataset with pretrained weights; seeded Gaussian draws
of the same shapes stand in for them (no dataset or checkpoint is used).

Distributions: X, dY ~ N(0, 1); W, B ~ N(0, 0.02^2); A ~ N(0, 1/d_in), i.e.
standard deviations 1, 0.02 and 1/sqrt(d_in).  Draw order per linear is
X, W, A, B, dY with numpy PCG64, each a float32 standard normal then scaled in
float32.  The float32 draws are what the oracle consumes; the GPU consumes
their bf16 round-to-nearest-even images (bf16 mode) or the float32 values
themselves (fp32 debug mode).
"""
from __future__ import annotations

import dataclasses
import math
from statistics import NormalDist

import numpy as np

__all__ = [
    "LinearShape", "Workload", "WORKLOADS", "make_linear_inputs", "make_norm_inputs", "codebook4_f32",
    "quantize4", "workload",
]


@dataclasses.dataclass(frozen=True)
class LinearShape:
    """One LoRA linear: tokens M, d_in K, d_out N, rank r, lora_alpha, seed."""
    name: str
    M: int
    K: int
    N: int
    r: int
    alpha: float
    seed: int
    quant4: bool = False

    @property
    def scale(self) -> float:
        """lora_alpha / r (the conventional LoRA scale)."""
        return self.alpha / self.r

    def flops(self) -> int:
        """Algorithmic FLOPs of one forward + backward (no dW, no recompute)."""
        M, K, N, r = self.M, self.K, self.N, self.r
        return 4 * M * N * K + 6 * M * r * (K + N)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    linears: tuple
    description: str

    def flops(self) -> int:
        return sum(l.flops() for l in self.linears)

    @property
    def tokens(self) -> int:
        return self.linears[0].M


def _decoder_layer() -> tuple:
    dims = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
            ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
    return tuple(LinearShape(f"decoder_{n}", 4096, k, nn, 64, 16.0, 1300 + i)
                 for i, (n, k, nn) in enumerate(dims))


WORKLOADS = {
    "tiny": Workload("tiny", (LinearShape("tiny", 64, 256, 256, 8, 32.0, 1000),),
                     "M=64, d_in=d_out=256, r=8, alpha=32"),
    "attn_proj_4096": Workload(
        "attn_proj_4096", (LinearShape("attn_proj_4096", 4096, 4096, 4096, 8, 32.0, 1001),),
        "M=4096 (batch 2 x seq 2048), d_in=d_out=4096, r=8, alpha=32"),
    "mlp_11008": Workload(
        "mlp_11008",
        (LinearShape("mlp_gate", 8192, 4096, 11008, 16, 32.0, 1200),
         LinearShape("mlp_up", 8192, 4096, 11008, 16, 32.0, 1201),
         LinearShape("mlp_down", 8192, 11008, 4096, 16, 32.0, 1202)),
        "gate/up 4096->11008 and down 11008->4096, M=8192, r=16, alpha=32"),
    "decoder_layer_r64": Workload(
        "decoder_layer_r64", _decoder_layer(),
        "seven LoRA linears q,k,v,o,gate,up,down, M=4096, r=64, alpha=16"),
    "qlora_28672": Workload(
        "qlora_28672", (LinearShape("qlora_28672", 2048, 8192, 28672, 16, 32.0, 1004, True),),
        "4-bit frozen W 8192->28672 (blocks of 64 along d_in, fp16 absmax), M=2048, r=16, alpha=32"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def make_linear_inputs(shape: LinearShape, *, M: int | None = None) -> dict:
    """Seeded float32 draws X[M,K], W[N,K], A[r,K], B[N,r], dY[M,N].

    ``M`` may be lowered to draw only the first rows of X and dY; the draw
    order then differs, so use it only for standalone small cases.
    """
    M = shape.M if M is None else M
    K, N, r = shape.K, shape.N, shape.r
    rng = np.random.Generator(np.random.PCG64(shape.seed))

    def normal(rows, cols, std):
        out = rng.standard_normal((rows, cols), dtype=np.float32)
        out *= np.float32(std)
        return out

    X = normal(M, K, 1.0)
    W = normal(N, K, 0.02)
    A = normal(r, K, 1.0 / math.sqrt(K))
    B = normal(N, r, 0.02)
    dY = normal(M, N, 1.0)
    return {"X": X, "W": W, "A": A, "B": B, "dY": dY}


# ----------------------------------------------------------------------------
# 4-bit weight format of the QLoRA workload (input preparation only).
#
# The frozen weight is stored as 4-bit codes in blocks of 64 along d_in with
# one fp16 absmax per block; the 16-entry codebook holds the normal quantiles
# Phi^-1((i + 0.5)/16) divided by Phi^-1(15.5/16), so that it spans [-1, 1].
# The pages only say the frozen weights are int4 and that dequantisation is
# fused into the matmul (page "Unsloth — 微调 2-5x 加速", section "核心要点",
# item 3); the concrete format is this workload's.  The codebook is passed to
# the library as an input array, like the codes and the absmax values.
# ----------------------------------------------------------------------------

QBLOCK = 64


def codebook4_f32() -> np.ndarray:
    """The 16 codebook values, float64 quantiles rounded once to float32."""
    nd = NormalDist()
    top = nd.inv_cdf(15.5 / 16.0)
    return np.array([nd.inv_cdf((i + 0.5) / 16.0) / top for i in range(16)], dtype=np.float32)


def quantize4(W: np.ndarray, codebook: np.ndarray | None = None):
    """Quantise W[N,K] (K % 64 == 0) to (codes[N,K/2] u8, absmax[N,K/64] fp16).

    absmax is the fp16 rounding of max|w| over each 64-block; each code is the
    nearest codebook entry to w/absmax (computed in float64 with the rounded
    absmax), ties to the lower index.  Element k even goes to the low nibble of
    byte k/2, k odd to the high nibble.
    """
    N, K = W.shape
    if K % QBLOCK:
        raise ValueError("K must be a multiple of 64")
    cb = (codebook4_f32() if codebook is None else codebook).astype(np.float64)
    if np.any(np.diff(cb) <= 0):
        raise ValueError("codebook must be strictly increasing")
    # nearest entry with ties to the lower index == count of midpoints strictly below y
    mids = (cb[:-1] + cb[1:]) * 0.5
    codes = np.empty((N, K // 2), dtype=np.uint8)
    absmax = np.empty((N, K // QBLOCK), dtype=np.float16)
    step = max(1, (1 << 22) // K)
    for r0 in range(0, N, step):
        w = W[r0:r0 + step].astype(np.float64)
        blocks = w.reshape(w.shape[0], K // QBLOCK, QBLOCK)
        am = np.abs(blocks).max(axis=2).astype(np.float16)
        absmax[r0:r0 + step] = am
        scale = am.astype(np.float64)[:, :, None]
        with np.errstate(invalid="ignore", divide="ignore"):
            y = np.where(scale > 0, blocks / np.where(scale > 0, scale, 1.0), 0.0)
        q = np.searchsorted(mids, y.reshape(w.shape[0], K), side="left").astype(np.uint8)
        codes[r0:r0 + step] = q[:, 0::2] | (q[:, 1::2] << 4)
    return codes, absmax


def make_norm_inputs(shape: LinearShape, *, M: int | None = None) -> dict:
    """Draws of make_linear_inputs for a linear behind an RMSNorm: X becomes a
    residual-stream input whose rows differ in magnitude (row m of X times
    exp(0.5 z_m), z_m ~ N(0, 1)), and the frozen norm weight g [K] ~ 1 + N(0,
    0.2^2) is added; both from a second PCG64 stream seeded seed + 7919, drawn
    in that order."""
    d = make_linear_inputs(shape, M=M)
    M = d["X"].shape[0]
    rng = np.random.Generator(np.random.PCG64(shape.seed + 7919))
    row = np.exp(rng.standard_normal(M, dtype=np.float32) * np.float32(0.5))
    d["X"] = d["X"] * row[:, None]
    d["g"] = np.float32(1.0) + rng.standard_normal(shape.K, dtype=np.float32) * np.float32(0.2)
    return d


def make_qlora_inputs(shape: LinearShape, *, M: int | None = None) -> dict:
    """Draws as make_linear_inputs, plus the 4-bit encoding of W."""
    d = make_linear_inputs(shape, M=M)
    cb = codebook4_f32()
    codes, absmax = quantize4(d["W"], cb)
    d.update(codes=codes, absmax=absmax, codebook=cb)
    return d


def device_inputs_torch(shape: LinearShape, device, dtype, seed: int):
    """Seeded device-side draws with the same distributions (benchmark inputs).

    Uses torch's generator on the device, so large workloads are drawn in
    milliseconds; these draws are not the numpy ones above.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    M, K, N, r = shape.M, shape.K, shape.N, shape.r

    def normal(rows, cols, std):
        t = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
        return (t * std).to(dtype)

    return {"X": normal(M, K, 1.0), "W": normal(N, K, 0.02), "A": normal(r, K, 1.0 / math.sqrt(K)),
            "B": normal(N, r, 0.02), "dY": normal(M, N, 1.0)}


def norm_weight_torch(K: int, device, dtype, seed: int):
    """Seeded device-side draw of an RMSNorm weight g [K] ~ 1 + N(0, 0.2^2)
    (benchmark inputs; not the numpy draw of make_norm_inputs)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (1.0 + 0.2 * torch.randn((K,), generator=g, device=device, dtype=torch.float32)).to(dtype)


def quantize4_torch(W):
    """Device-side version of quantize4 for benchmark inputs (float32 arithmetic).

    Returns codes [N, K/2] uint8, absmax [N, K/64] fp16 bit patterns as int16,
    and the float32 codebook, all on W's device.
    """
    import torch
    N, K = W.shape
    cb = torch.from_numpy(codebook4_f32()).to(W.device)
    mids = ((cb[:-1].double() + cb[1:].double()) * 0.5).float()
    blocks = W.float().reshape(N, K // QBLOCK, QBLOCK)
    am = blocks.abs().amax(dim=2).to(torch.float16)
    scale = am.float().unsqueeze(2)
    y = torch.where(scale > 0, blocks / torch.where(scale > 0, scale, torch.ones_like(scale)),
                    torch.zeros_like(blocks))
    q = torch.bucketize(y.reshape(N, K), mids).to(torch.uint8)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).contiguous()
    return {"codes": codes, "absmax": am.view(torch.int16).contiguous(), "codebook": cb}
