"""ctypes loader for liblora_linear.so (the C ABI in include/lora_linear.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# LORA_LINEAR_LIB selects another build of the same library (e.g. one with the
# host code instrumented by a sanitizer); the in-tree build is the default.
LIB_PATH = os.environ.get("LORA_LINEAR_LIB") or os.path.join(HERE, "liblora_linear.so")

LORA_OK = 0
LORA_ERR_INVALID_ARG = 1
LORA_ERR_UNSUPPORTED = 2
LORA_ERR_MISALIGNED = 3
LORA_ERR_WORKSPACE_TOO_SMALL = 4
LORA_ERR_HIP = 5

LORA_DTYPE_BF16 = 0
LORA_DTYPE_F32 = 1

LORA_FLAG_ACCUM_GRADS = 0x1
LORA_FLAG_W_TRANSPOSED = 0x2
LORA_NOALLOC_SCRATCH_BYTES = 128 << 20
LORA_MAX_MEMBERS = 8
LORA_MAX_GROUP_RANK = 192

EXPORTED = (
    "lora_linear_workspace_size", "lora_linear_fwd", "lora_linear_bwd", "lora_linear_bwd_noalloc",
    "lora_qlinear_fwd", "lora_qlinear_bwd", "lora_dequant4", "lora_merge",
    "lora_linear_buffer_ranges", "lora_group_workspace_size", "lora_group_fwd", "lora_group_bwd",
    "lora_transpose_weight", "lora_fold_norm_weight", "lora_norm_linear_workspace_size", "lora_norm_linear_fwd", "lora_norm_linear_bwd",
    "lora_norm_group_workspace_size", "lora_norm_group_fwd", "lora_norm_group_bwd",
    "lora_tune_linear", "lora_tuner_lookup", "lora_tuner_save", "lora_tuner_load", "lora_tuner_clear",
    "lora_set_kernel_timer", "lora_status_string", "lora_last_error",
)

# void (*)(void* user, const char* kernel, void* stream, void** start_event, void** stop_event)
KERNEL_TIMER = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_char_p, ctypes.c_void_p,
                                ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p))


class LoraLinearDesc(ctypes.Structure):
    """Mirror of struct lora_linear_desc."""
    _fields_ = [
        ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("N", ctypes.c_int64), ("r", ctypes.c_int64),
        ("alpha", ctypes.c_float), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
    ]


class LoraGroupDesc(ctypes.Structure):
    """Mirror of struct lora_group_desc."""
    _fields_ = [
        ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("r", ctypes.c_int64), ("alpha", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("n_members", ctypes.c_int32),
        ("N", ctypes.c_int64 * LORA_MAX_MEMBERS),
    ]


class LoraTunedConfig(ctypes.Structure):
    """Mirror of struct lora_tuned_config."""
    _fields_ = [("fwd_split", ctypes.c_int32), ("bwd_split", ctypes.c_int32), ("rank_div", ctypes.c_int32),
                ("z_div_fwd", ctypes.c_int32), ("z_div_bwd", ctypes.c_int32), ("fwd_us", ctypes.c_float),
                ("bwd_us", ctypes.c_float), ("default_fwd_us", ctypes.c_float), ("default_bwd_us", ctypes.c_float)]


class LoraBufferRange(ctypes.Structure):
    """Mirror of struct lora_buffer_range."""
    _fields_ = [("kernel", ctypes.c_char_p), ("operand", ctypes.c_char_p), ("bytes", ctypes.c_uint64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the library once and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first (python -m lora_linear_layer_amd.build); "
            "the LoRA layer has no non-HIP implementation")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    dp = ctypes.POINTER(LoraLinearDesc)
    gp = ctypes.POINTER(LoraGroupDesc)
    sig = {
        "lora_linear_workspace_size": [dp, ctypes.POINTER(sz)],
        "lora_linear_fwd": [dp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lora_linear_bwd": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lora_linear_bwd_noalloc": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "lora_qlinear_fwd": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lora_qlinear_bwd": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lora_dequant4": [vp, vp, vp, i64, i64, i32, vp, vp],
        "lora_merge": [dp, vp, vp, vp, vp, i32, vp],
        "lora_linear_buffer_ranges": [dp, i32, ctypes.POINTER(LoraBufferRange), i32, ctypes.POINTER(i32)],
        "lora_group_workspace_size": [gp, ctypes.POINTER(sz)],
        "lora_tune_linear": [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i32,
                             ctypes.POINTER(LoraTunedConfig)],
        "lora_tuner_lookup": [ctypes.c_char_p, i32, dp, i32, ctypes.POINTER(LoraTunedConfig), ctypes.POINTER(i32)],
        "lora_tuner_save": [ctypes.c_char_p],
        "lora_tuner_load": [ctypes.c_char_p],
        "lora_group_fwd": [gp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lora_group_bwd": [gp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lora_fold_norm_weight": [vp, vp, i64, i64, vp, vp],
        "lora_transpose_weight": [vp, i64, i64, vp, vp],
        "lora_norm_linear_workspace_size": [dp, ctypes.POINTER(sz)],
        "lora_norm_linear_fwd": [dp, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lora_norm_linear_bwd": [dp, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lora_norm_group_workspace_size": [gp, ctypes.POINTER(sz)],
        "lora_norm_group_fwd": [gp, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lora_norm_group_bwd": [gp, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.lora_set_kernel_timer.argtypes = [KERNEL_TIMER, ctypes.c_void_p]
    lib.lora_set_kernel_timer.restype = None
    lib.lora_tuner_clear.argtypes = []
    lib.lora_tuner_clear.restype = None
    lib.lora_status_string.argtypes = [ctypes.c_int]
    lib.lora_status_string.restype = ctypes.c_char_p
    lib.lora_last_error.argtypes = []
    lib.lora_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib
