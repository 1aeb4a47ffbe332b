"""torch.autograd glue over the C ABI (a drop-in LoRA linear for training loops).

The module mirrors the pages' description of the accelerated layer: the
frozen linear is replaced by a module whose forward and backward call the
fused kernels directly, without autograd tracing the adapter products (page
"UnSloth加速库集成：编译级优化带来的性能飞跃", section "技术四：无缝兼容生态",
and page "ms-swift高效微调组合：LoRA+UnSloth提速实践", section 1.2).
Only memory allocation and stream handling come from PyTorch.
"""
from __future__ import annotations

import math

import torch

from . import api
from ._lib import LORA_DTYPE_BF16, LORA_DTYPE_F32, LORA_FLAG_W_TRANSPOSED

_DTYPES = {torch.bfloat16: LORA_DTYPE_BF16, torch.float32: LORA_DTYPE_F32}


def _desc(M, K, N, r, alpha, dtype) -> api.Desc:
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype} (bfloat16 or float32)")
    return api.Desc(M, K, N, r, float(alpha), _DTYPES[dtype])


def _same(x, **ts):
    """x and the adapter (and 16-bit weight) tensors share x's dtype and device."""
    for name, t in ts.items():
        if t.dtype != x.dtype:
            raise TypeError(f"{name} has dtype {t.dtype} but the input has {x.dtype}; the layer computes in one "
                            "dtype (cast the input, or build the layer in the input's dtype)")
        if t.device != x.device:
            raise ValueError(f"{name} is on {t.device} but the input is on {x.device}")


class LoraLinearFunction(torch.autograd.Function):
    """H = X W^T + (alpha/r) (X A^T) B^T with W frozen (no gradient for W).

    Wt (optional, bf16 [in, out]): W^T made once from the frozen weight; the
    backward then reads it (LORA_FLAG_W_TRANSPOSED) instead of W, with
    bit-identical results."""

    @staticmethod
    def forward(ctx, x, W, A, B, alpha, Wt=None):
        lead = x.shape[:-1]
        K = x.shape[-1]
        X = x.reshape(-1, K).contiguous()
        N, r = B.shape
        _same(X, W=W, A=A, B=B)
        desc = _desc(X.shape[0], K, N, r, alpha, X.dtype)
        H = torch.empty((X.shape[0], N), dtype=X.dtype, device=X.device)
        U = torch.empty((X.shape[0], r), dtype=torch.float32, device=X.device)
        ws = torch.empty(max(api.lora_linear_workspace_size(desc), 1), dtype=torch.uint8, device=X.device)
        api.lora_linear_fwd(desc, X, W.contiguous(), A.contiguous(), B.contiguous(), H, U, ws=ws)
        if Wt is not None:
            _same(X, Wt=Wt)
            if tuple(Wt.shape) != (K, N):
                raise ValueError(f"Wt has shape {tuple(Wt.shape)}, expected {(K, N)}")
            desc = api.Desc(desc.M, desc.K, desc.N, desc.r, desc.alpha, desc.dtype,
                            desc.flags | LORA_FLAG_W_TRANSPOSED)
            W = Wt
        ctx.save_for_backward(X, W, A, B, U)
        ctx.desc = desc
        ctx.lead = lead
        return H.reshape(*lead, N)

    @staticmethod
    def backward(ctx, dH):
        X, W, A, B, U = ctx.saved_tensors
        desc = ctx.desc
        dY = dH.reshape(-1, desc.N).to(X.dtype).contiguous()
        dX = torch.empty_like(X) if ctx.needs_input_grad[0] else None
        dA = torch.empty_like(A)
        dB = torch.empty_like(B)
        ws = torch.empty(max(api.lora_linear_workspace_size(desc), 1), dtype=torch.uint8, device=X.device)
        api.lora_linear_bwd(desc, dY, X, W.contiguous(), A.contiguous(), B.contiguous(), U, dX, dA, dB, ws=ws)
        dx = dX.reshape(*ctx.lead, desc.K) if dX is not None else None
        return dx, None, dA, dB, None, None


class QLoraLinearFunction(torch.autograd.Function):
    """As LoraLinearFunction with W given by 4-bit codes, fp16 absmax and a codebook."""

    @staticmethod
    def forward(ctx, x, Wq, absmax, codebook, A, B, alpha):
        lead = x.shape[:-1]
        K = x.shape[-1]
        X = x.reshape(-1, K).contiguous()
        N, r = B.shape
        _same(X, A=A, B=B)
        desc = _desc(X.shape[0], K, N, r, alpha, X.dtype)
        H = torch.empty((X.shape[0], N), dtype=X.dtype, device=X.device)
        U = torch.empty((X.shape[0], r), dtype=torch.float32, device=X.device)
        ws = torch.empty(max(api.lora_linear_workspace_size(desc), 1), dtype=torch.uint8, device=X.device)
        api.lora_qlinear_fwd(desc, X, Wq, absmax, codebook, A.contiguous(), B.contiguous(), H, U, ws=ws)
        ctx.save_for_backward(X, Wq, absmax, codebook, A, B, U)
        ctx.desc = desc
        ctx.lead = lead
        return H.reshape(*lead, N)

    @staticmethod
    def backward(ctx, dH):
        X, Wq, absmax, codebook, A, B, U = ctx.saved_tensors
        desc = ctx.desc
        dY = dH.reshape(-1, desc.N).to(X.dtype).contiguous()
        dX = torch.empty_like(X) if ctx.needs_input_grad[0] else None
        dA = torch.empty_like(A)
        dB = torch.empty_like(B)
        ws = torch.empty(max(api.lora_linear_workspace_size(desc), 1), dtype=torch.uint8, device=X.device)
        api.lora_qlinear_bwd(desc, dY, X, Wq, absmax, codebook, A.contiguous(), B.contiguous(), U, dX, dA, dB, ws=ws)
        dx = dX.reshape(*ctx.lead, desc.K) if dX is not None else None
        return dx, None, None, None, dA, dB, None


class LoraLinear(torch.nn.Module):
    """Frozen W [out, in] plus trainable A [r, in], B [out, r]; s = alpha / r.

    B starts at zero, so the layer starts as the frozen linear.  With
    keep_transposed_weight (bf16 on a GPU) the module also holds W^T as a
    buffer, made once, and its backward reads that (faster input-gradient GEMM,
    bit-identical results, one more copy of W in memory); call
    refresh_transposed_weight() after changing the weight.
    """

    def __init__(self, in_features, out_features, r, alpha, weight=None, dtype=torch.bfloat16, device=None,
                 keep_transposed_weight=False):
        super().__init__()
        self.r, self.alpha = r, float(alpha)
        w = weight if weight is not None else torch.empty(out_features, in_features, dtype=dtype, device=device)
        self.weight = torch.nn.Parameter(w.to(dtype=dtype, device=device), requires_grad=False)
        self.lora_A = torch.nn.Parameter(torch.empty(r, in_features, dtype=dtype, device=device))
        self.lora_B = torch.nn.Parameter(torch.zeros(out_features, r, dtype=dtype, device=device))
        torch.nn.init.normal_(self.lora_A, std=1.0 / math.sqrt(in_features))
        wt = torch.empty(in_features, out_features, dtype=dtype, device=device) if keep_transposed_weight else None
        self.register_buffer("weight_t", wt, persistent=False)   # derived from weight: not saved
        if keep_transposed_weight:
            self.refresh_transposed_weight()

    @torch.no_grad()
    def refresh_transposed_weight(self):
        """weight_t = weight^T (lora_transpose_weight)."""
        if self.weight_t is None:
            raise RuntimeError("the module was built without keep_transposed_weight")
        api.lora_transpose_weight(self.weight.contiguous(), self.weight_t)

    def forward(self, x):
        # the layer computes in its parameters' dtype (e.g. float32 activations
        # from an autocast region are converted to bf16 here)
        if x.dtype != self.weight.dtype:
            x = x.to(self.weight.dtype)
        return LoraLinearFunction.apply(x, self.weight, self.lora_A, self.lora_B, self.alpha, self.weight_t)

    @torch.no_grad()
    def merged_weight(self, sign: int = 1) -> torch.Tensor:
        """W + sign * s * B A as a new tensor (sign +1: the adapter folded in for
        deployment, page "ms-swift框架下UnSloth与Liger-Kernel优化实战", section
        "设计权衡与最佳实践", item 4; sign -1 removes it again)."""
        W = self.weight.contiguous()
        desc = _desc(1, W.shape[1], W.shape[0], self.r, self.alpha, W.dtype)
        out = torch.empty_like(W)
        api.lora_merge(desc, W, self.lora_A.contiguous(), self.lora_B.contiguous(), out, sign)
        return out
