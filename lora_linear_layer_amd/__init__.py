"""Fused LoRA linear layer for AMD MI355X (gfx950): HIP kernels behind a C ABI.

The Python names mirror the C entry points in include/lora_linear.h; the
autograd wrappers live in lora_linear_layer_amd.layer.
"""
from ._lib import (LIB_PATH, LORA_DTYPE_BF16, LORA_DTYPE_F32, LORA_FLAG_ACCUM_GRADS,  # noqa: F401
                   LORA_FLAG_W_TRANSPOSED, LORA_NOALLOC_SCRATCH_BYTES, load)
from .api import (Desc, GroupDesc, LoraError, lora_dequant4, lora_group_bwd, lora_group_fwd,  # noqa: F401
                  lora_group_workspace_size, lora_linear_buffer_ranges, lora_linear_bwd,
                  lora_linear_bwd_noalloc, lora_transpose_weight, lora_fold_norm_weight, lora_norm_linear_workspace_size,
                  lora_norm_linear_fwd, lora_norm_linear_bwd, lora_norm_group_workspace_size,
                  lora_norm_group_fwd, lora_norm_group_bwd,
                  lora_linear_fwd, lora_linear_workspace_size, lora_merge, lora_qlinear_bwd, lora_qlinear_fwd,
                  lora_set_kernel_timer, lora_tune_linear, lora_tuner_clear, lora_tuner_load,
                  lora_tuner_lookup, lora_tuner_save)

__all__ = [
    "Desc", "GroupDesc", "LoraError", "lora_linear_workspace_size", "lora_linear_fwd", "lora_linear_bwd",
    "lora_group_workspace_size", "lora_group_fwd", "lora_group_bwd",
    "lora_linear_bwd_noalloc", "LORA_NOALLOC_SCRATCH_BYTES",
    "lora_transpose_weight", "lora_fold_norm_weight", "lora_norm_linear_workspace_size", "lora_norm_linear_fwd", "lora_norm_linear_bwd",
    "lora_norm_group_workspace_size", "lora_norm_group_fwd", "lora_norm_group_bwd",
    "lora_qlinear_fwd", "lora_qlinear_bwd", "lora_dequant4", "lora_merge", "lora_linear_buffer_ranges",
    "lora_set_kernel_timer", "lora_tune_linear", "lora_tuner_lookup", "lora_tuner_save", "lora_tuner_load",
    "lora_tuner_clear", "load", "LIB_PATH",
    "LORA_DTYPE_BF16", "LORA_DTYPE_F32", "LORA_FLAG_ACCUM_GRADS", "LORA_FLAG_W_TRANSPOSED",
]
