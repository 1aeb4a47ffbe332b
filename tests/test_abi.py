"""C ABI contract tests that need no GPU.

The library must load, export every function include/lora_linear.h declares,
and reject bad arguments with the documented status before any HIP call.
Every call below fails validation, so nothing is ever enqueued.
"""
import ctypes
import os
import re

import pytest

import lora_linear_layer_amd as lla
from lora_linear_layer_amd import _lib
from lora_linear_layer_amd._lib import LoraLinearDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_linear.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")

ALIGNED = 0x10000          # a fake, 16-byte aligned address; never dereferenced
MISALIGNED = 0x10008


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_\w+)\s*\(", text)))


def test_header_declares_expected_api():
    names = header_functions()
    for n in ("lora_linear_fwd", "lora_linear_bwd", "lora_qlinear_fwd", "lora_qlinear_bwd",
              "lora_dequant4", "lora_merge", "lora_linear_workspace_size", "lora_status_string",
              "lora_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
    assert set(header_functions()) == set(_lib.EXPORTED)


def test_struct_layout_matches_header():
    assert ctypes.sizeof(LoraLinearDesc) == 4 * 8 + 4 + 4 + 4 + 4  # 4 x int64, float, int32, uint32, pad
    assert LoraLinearDesc.alpha.offset == 32 and LoraLinearDesc.flags.offset == 40


def lib():
    return _lib.load()


def desc(**kw):
    d = dict(M=64, K=256, N=256, r=8, alpha=32.0, dtype=0, flags=0)
    d.update(kw)
    return LoraLinearDesc(d["M"], d["K"], d["N"], d["r"], d["alpha"], d["dtype"], d["flags"])


def ws_size(d):
    out = ctypes.c_size_t()
    st = lib().lora_linear_workspace_size(ctypes.byref(d), ctypes.byref(out))
    return st, out.value


def fwd(d, X=ALIGNED, W=ALIGNED + 0x100, A=ALIGNED + 0x200, B=ALIGNED + 0x300, H=ALIGNED + 0x400,
        U=None, ws=None, ws_bytes=0):
    return lib().lora_linear_fwd(ctypes.byref(d) if d is not None else None, X, W, A, B, H, U, ws, ws_bytes, None)


def bwd(d, dY=ALIGNED, X=ALIGNED + 0x100, W=ALIGNED + 0x200, A=ALIGNED + 0x300, B=ALIGNED + 0x400,
        U=None, dX=ALIGNED + 0x500, dA=ALIGNED + 0x600, dB=ALIGNED + 0x700, ws=None, ws_bytes=0):
    return lib().lora_linear_bwd(ctypes.byref(d), dY, X, W, A, B, U, dX, dA, dB, ws, ws_bytes, None)


def test_status_strings():
    L = lib()
    for code in range(6):
        assert L.lora_status_string(code)
    assert L.lora_status_string(99) == b"unknown status"


@pytest.mark.parametrize("field,value", [("M", 0), ("K", -8), ("N", 0), ("r", 0)])
def test_nonpositive_sizes(field, value):
    d = desc(**{field: value})
    assert fwd(d) == _lib.LORA_ERR_INVALID_ARG
    assert ws_size(d)[0] == _lib.LORA_ERR_INVALID_ARG
    assert b"positive" in lib().lora_last_error()


def test_null_desc_and_bad_dtype_and_flags():
    assert fwd(None) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(desc(dtype=7)) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(desc(flags=0x80)) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(desc(alpha=float("nan"))) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(desc(alpha=float("inf"))) == _lib.LORA_ERR_INVALID_ARG


def test_unsupported_shapes():
    assert fwd(desc(r=129)) == _lib.LORA_ERR_UNSUPPORTED
    assert fwd(desc(K=260)) == _lib.LORA_ERR_UNSUPPORTED
    assert fwd(desc(N=12)) == _lib.LORA_ERR_UNSUPPORTED
    assert fwd(desc(M=1 << 20, K=1 << 12)) == _lib.LORA_ERR_UNSUPPORTED      # 2^32 elements
    d = desc(K=96)
    assert lib().lora_qlinear_fwd(ctypes.byref(d), ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED,
                                  None, None, 0, None) == _lib.LORA_ERR_UNSUPPORTED


def test_null_and_misaligned_pointers():
    d = desc()
    assert fwd(d, X=None) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(d, H=None) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(d, W=MISALIGNED) == _lib.LORA_ERR_MISALIGNED
    assert fwd(d, U=MISALIGNED) == _lib.LORA_ERR_MISALIGNED
    assert bwd(d, dA=None) == _lib.LORA_ERR_INVALID_ARG
    assert bwd(d, dX=MISALIGNED) == _lib.LORA_ERR_MISALIGNED


def test_aliasing_rejected():
    d = desc()
    assert fwd(d, H=ALIGNED) == _lib.LORA_ERR_INVALID_ARG          # H aliases X
    assert b"aliases" in lib().lora_last_error()
    assert bwd(d, dA=ALIGNED + 0x700) == _lib.LORA_ERR_INVALID_ARG  # dA aliases dB


def test_workspace_checks():
    d = desc()
    st, need = ws_size(d)
    assert st == _lib.LORA_OK and need > 0
    assert fwd(d, ws=ALIGNED + 0x1000, ws_bytes=need - 1) == _lib.LORA_ERR_WORKSPACE_TOO_SMALL
    assert bwd(d, ws=None, ws_bytes=0) == _lib.LORA_ERR_WORKSPACE_TOO_SMALL
    assert bwd(d, ws=ALIGNED + 0x1008, ws_bytes=need) == _lib.LORA_ERR_MISALIGNED
    assert bwd(d, ws=None, ws_bytes=need) == _lib.LORA_ERR_INVALID_ARG


def test_workspace_grows_with_problem():
    small = ws_size(desc())[1]
    big = ws_size(desc(M=4096, K=4096, N=4096))[1]
    f32 = ws_size(desc(M=4096, K=4096, N=4096, dtype=1))[1]
    assert big > small and f32 < big


def test_dequant4_validation():
    L = lib()
    assert L.lora_dequant4(ALIGNED, ALIGNED + 0x100, ALIGNED + 0x200, 0, 64, 0, ALIGNED + 0x300, None) == \
        _lib.LORA_ERR_INVALID_ARG
    assert L.lora_dequant4(ALIGNED, ALIGNED + 0x100, ALIGNED + 0x200, 8, 96, 0, ALIGNED + 0x300, None) == \
        _lib.LORA_ERR_UNSUPPORTED
    assert L.lora_dequant4(ALIGNED, ALIGNED + 0x100, ALIGNED + 0x200, 8, 64, 5, ALIGNED + 0x300, None) == \
        _lib.LORA_ERR_INVALID_ARG
    assert L.lora_dequant4(ALIGNED, ALIGNED + 0x100, None, 8, 64, 0, ALIGNED + 0x300, None) == \
        _lib.LORA_ERR_INVALID_ARG
    assert L.lora_dequant4(ALIGNED, ALIGNED + 0x100, ALIGNED + 0x200, 8, 64, 0, ALIGNED, None) == \
        _lib.LORA_ERR_INVALID_ARG


def test_merge_validation():
    """lora_merge: W_out may equal W (in place, not checked here: that call would
    launch), but must not overlap W otherwise, nor A or B; sign is +1 or -1;
    r <= 128, K % 8 == 0."""
    L = lib()
    W, A, B, O = ALIGNED, ALIGNED + 0x1000, ALIGNED + 0x2000, ALIGNED + 0x3000
    d = desc(M=1, K=64, N=32, r=8)
    ok_args = (W, A, B, O)
    assert L.lora_merge(None, *ok_args, 1, None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_merge(ctypes.byref(d), *ok_args, 0, None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_merge(ctypes.byref(d), *ok_args, 2, None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_merge(ctypes.byref(d), W, A, B, A, 1, None) == _lib.LORA_ERR_INVALID_ARG      # W_out is A
    assert L.lora_merge(ctypes.byref(d), W, A, B, B, -1, None) == _lib.LORA_ERR_INVALID_ARG     # W_out is B
    assert L.lora_merge(ctypes.byref(d), W, None, B, O, 1, None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_merge(ctypes.byref(d), W, A, B, MISALIGNED, 1, None) == _lib.LORA_ERR_MISALIGNED
    assert L.lora_merge(ctypes.byref(desc(M=1, K=60, N=32, r=8)), *ok_args, 1, None) == _lib.LORA_ERR_UNSUPPORTED
    assert L.lora_merge(ctypes.byref(desc(M=1, K=64, N=32, r=129)), *ok_args, 1, None) == _lib.LORA_ERR_UNSUPPORTED
    assert L.lora_merge(ctypes.byref(desc(M=1, K=64, N=0, r=8)), *ok_args, 1, None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_merge(ctypes.byref(desc(M=1, K=64, N=32, r=8, dtype=7)), *ok_args, 1, None) == \
        _lib.LORA_ERR_INVALID_ARG
    # W is 32 x 64 bf16 = 4 KB: a W_out 16 bytes past W overlaps it, as does one inside A's range
    assert L.lora_merge(ctypes.byref(d), W, A, B, W + 16, 1, None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_merge(ctypes.byref(d), W, A, B, A - 0x800, 1, None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_merge(ctypes.byref(d), W, A, B, B + 0x100, 1, None) == _lib.LORA_ERR_INVALID_ARG


def test_python_binding_raises():
    with pytest.raises(lla.LoraError) as ei:
        lla.lora_linear_workspace_size(lla.Desc(0, 8, 8, 1, 1.0))
    assert ei.value.status == _lib.LORA_ERR_INVALID_ARG


# ------------------------------------------------------------ buffer ranges
MAX_RANGE = (1 << 31) - 1

# descriptors at the edges of the supported range: 16-bit inputs above 2 GB,
# the largest K and N, the largest rank, tiny K with many tokens
EDGE_DESCS = [
    dict(M=(1 << 30) // 4096 + 64, K=4096, N=64, r=32),          # X just over 2 GB (2^30 + 2^18 elements)
    dict(M=(1 << 31) // 4096 - 1, K=4096, N=4096, r=128),        # X and dY just under 4 GB
    dict(M=(1 << 31) // 4096 - 1, K=4096, N=4096, r=8),
    dict(M=1023, K=1 << 21, N=1000, r=128),                      # K at 2^21
    dict(M=1000, K=960, N=1 << 21, r=128),                       # N at 2^21
    dict(M=(1 << 28) - 8, K=8, N=8, r=7),                        # 2^28 tokens: M r just under 2^31
    dict(M=(1 << 24) - 1, K=128, N=128, r=128),                  # M r just under 2^31 at the top rank
    dict(M=(1 << 25) - 1, K=64, N=64, r=64),
    dict(M=65, K=(1 << 21) - 64, N=1000, r=100),
]


@pytest.mark.parametrize("quant", [False, True])
@pytest.mark.parametrize("kw", EDGE_DESCS)
def test_buffer_ranges_fit_32_bits(kw, quant):
    """Every buffer resource the bf16 kernels build stays within the 2^31 - 1
    bytes its range field can describe, so no valid load reads zeros."""
    if quant and kw["K"] % 64:
        pytest.skip("4-bit entry points need K % 64 == 0")
    d = lla.Desc(kw["M"], kw["K"], kw["N"], kw["r"], 16.0)
    ranges = lla.lora_linear_buffer_ranges(d, quant)
    assert ranges, "no resources listed"
    kernels = {k for k, _, _ in ranges}
    assert any("lora_gemm (forward)" in k for k in kernels) and any("lora_gemm (dX)" in k for k in kernels)
    assert any("rank_stream" in k for k in kernels) and any("rank_z_lds" in k for k in kernels)
    too_big = [(k, o, b) for k, o, b in ranges if not 0 < b <= MAX_RANGE]
    assert not too_big, too_big


def test_buffer_ranges_x_over_2gb_is_blockwise():
    """X of 2^30 + 2^18 bf16 elements (2.15 GB): the streamed U pass addresses
    it in 128-row blocks (1 MB each), not as one resource over all of X."""
    M, K = (1 << 30) // 4096 + 64, 4096
    ranges = lla.lora_linear_buffer_ranges(lla.Desc(M, K, 64, 32, 16.0))
    y = [b for k, o, b in ranges if k.startswith("rank_z_lds (U") and o.startswith("Y block")]
    assert y == [128 * K * 2]
    assert 2 * M * K > MAX_RANGE


def test_buffer_ranges_f32_mode_builds_none():
    assert lla.lora_linear_buffer_ranges(lla.Desc(64, 256, 256, 8, 32.0, lla.LORA_DTYPE_F32)) == []


def test_buffer_ranges_rejects_bad_descriptor():
    with pytest.raises(lla.LoraError):
        lla.lora_linear_buffer_ranges(lla.Desc(64, 250, 256, 8, 32.0))
    with pytest.raises(lla.LoraError):
        lla.lora_linear_buffer_ranges(lla.Desc(64, 96, 256, 8, 32.0), quant=True)


def test_kernel_timer_set_and_clear():
    """The timer can be set and removed; a call refused by validation enqueues
    nothing, so the timer is never asked for events."""
    seen = []
    lla.lora_set_kernel_timer(lambda k, s: seen.append(k))
    try:
        assert fwd(desc(K=250)) == _lib.LORA_ERR_UNSUPPORTED
    finally:
        lla.lora_set_kernel_timer(None)
    assert seen == []


# ------------------------------------------------------------ grouped linears
def test_group_desc_layout_and_checks():
    from lora_linear_layer_amd._lib import LoraGroupDesc
    assert ctypes.sizeof(LoraGroupDesc) == 3 * 8 + 4 + 4 + 4 + 4 + 8 * 8     # pad after n_members
    assert LoraGroupDesc.N.offset == 40
    ok = lla.GroupDesc(64, 256, (256, 64, 64), 16, 32.0)
    assert lla.lora_group_workspace_size(ok) > 0
    for bad, status in ((lla.GroupDesc(64, 256, (256, 64), 100, 16.0), _lib.LORA_ERR_UNSUPPORTED),   # rank 200
                        (lla.GroupDesc(64, 256, (256, 60), 16, 16.0), _lib.LORA_ERR_UNSUPPORTED),    # N % 8
                        (lla.GroupDesc(64, 250, (256,), 16, 16.0), _lib.LORA_ERR_UNSUPPORTED),       # K % 8
                        (lla.GroupDesc(64, 256, (256, 0), 16, 16.0), _lib.LORA_ERR_INVALID_ARG),
                        (lla.GroupDesc(64, 256, (256,), 16, 16.0, lla.LORA_DTYPE_F32), _lib.LORA_ERR_UNSUPPORTED)):
        with pytest.raises(lla.LoraError) as e:
            lla.lora_group_workspace_size(bad)
        assert e.value.status == status
    d = lla.GroupDesc(64, 256, (256,), 16, 16.0).c()
    d.n_members = 9
    out = ctypes.c_size_t()
    assert lib().lora_group_workspace_size(ctypes.byref(d), ctypes.byref(out)) == _lib.LORA_ERR_INVALID_ARG


def test_group_calls_validate_before_any_hip_call():
    d = lla.GroupDesc(64, 256, (256, 64), 16, 32.0).c()
    need = lla.lora_group_workspace_size(lla.GroupDesc(64, 256, (256, 64), 16, 32.0))
    L = lib()
    assert L.lora_group_fwd(ctypes.byref(d), ALIGNED, ALIGNED + 0x100, ALIGNED + 0x200, ALIGNED + 0x300, None, None,
                            ALIGNED + 0x500, need, None) == _lib.LORA_ERR_INVALID_ARG              # H NULL
    assert L.lora_group_fwd(ctypes.byref(d), MISALIGNED, ALIGNED + 0x100, ALIGNED + 0x200, ALIGNED + 0x300,
                            ALIGNED + 0x400, None, ALIGNED + 0x500, need, None) == _lib.LORA_ERR_MISALIGNED
    assert L.lora_group_fwd(ctypes.byref(d), ALIGNED, ALIGNED + 0x100, ALIGNED + 0x200, ALIGNED + 0x300,
                            ALIGNED + 0x400, None, ALIGNED + 0x500, need - 1, None) == _lib.LORA_ERR_WORKSPACE_TOO_SMALL
    assert L.lora_group_bwd(ctypes.byref(d), ALIGNED, ALIGNED + 0x100, ALIGNED + 0x200, ALIGNED + 0x300,
                            ALIGNED + 0x400, None, ALIGNED, ALIGNED + 0x600, ALIGNED + 0x700, ALIGNED + 0x800, need,
                            None) == _lib.LORA_ERR_INVALID_ARG                                       # dX aliases dY


def test_norm_calls_validate_before_any_hip_call():
    """RMSNorm entry points: bf16 only, eps >= 0 and finite, the usual pointer,
    alias and workspace checks, all before anything is enqueued."""
    L = lib()
    desc = lla.Desc(64, 256, 128, 8, 16.0)
    d = desc.c()
    need = lla.lora_norm_linear_workspace_size(desc)
    assert need > lla.lora_linear_workspace_size(desc)          # + inv [M] and A diag(g) [r][K]
    f32 = lla.Desc(64, 256, 128, 8, 16.0, lla.LORA_DTYPE_F32).c()
    out = ctypes.c_size_t()
    assert L.lora_norm_linear_workspace_size(ctypes.byref(f32), ctypes.byref(out)) == _lib.LORA_ERR_UNSUPPORTED
    p = [ALIGNED + 0x100 * i for i in range(16)]
    fwd = L.lora_norm_linear_fwd
    assert fwd(ctypes.byref(f32), 1e-6, *p[:6], None, None, p[9], need, None) == _lib.LORA_ERR_UNSUPPORTED
    assert fwd(ctypes.byref(d), -1e-6, *p[:6], None, None, p[9], need, None) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(ctypes.byref(d), float("nan"), *p[:6], None, None, p[9], need, None) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(ctypes.byref(d), 1e-6, p[0], None, *p[2:6], None, None, p[9], need, None) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(ctypes.byref(d), 1e-6, *p[:5], MISALIGNED, None, None, p[9], need, None) == _lib.LORA_ERR_MISALIGNED
    assert fwd(ctypes.byref(d), 1e-6, *p[:6], None, p[0], p[9], need, None) == _lib.LORA_ERR_INVALID_ARG  # inv = X
    assert fwd(ctypes.byref(d), 1e-6, *p[:6], None, None, p[9], need - 1, None) == _lib.LORA_ERR_WORKSPACE_TOO_SMALL
    bwd = L.lora_norm_linear_bwd
    assert bwd(ctypes.byref(d), 1e-6, *p[:6], None, None, p[1], p[7], p[8], p[9], need,
               None) == _lib.LORA_ERR_INVALID_ARG                                                  # dX aliases X
    assert bwd(ctypes.byref(d), 1e-6, *p[:6], None, None, p[6], None, p[8], p[9], need,
               None) == _lib.LORA_ERR_INVALID_ARG                                                  # dA NULL
    assert L.lora_fold_norm_weight(p[0], p[1], 128, 252, p[2], None) == _lib.LORA_ERR_UNSUPPORTED  # K % 8
    assert L.lora_fold_norm_weight(p[0], p[1], 0, 256, p[2], None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_fold_norm_weight(p[0], p[1], 128, 256, p[1], None) == _lib.LORA_ERR_INVALID_ARG  # W_out = g
    assert L.lora_fold_norm_weight(MISALIGNED, p[1], 128, 256, p[2], None) == _lib.LORA_ERR_MISALIGNED


def test_norm_group_calls_validate_before_any_hip_call():
    L = lib()
    gd = lla.GroupDesc(64, 256, (256, 64), 16, 32.0)
    d = gd.c()
    need = lla.lora_norm_group_workspace_size(gd)
    assert need > lla.lora_group_workspace_size(gd)
    p = [ALIGNED + 0x100 * i for i in range(16)]
    fwd, bwd = L.lora_norm_group_fwd, L.lora_norm_group_bwd
    assert fwd(ctypes.byref(d), -1.0, *p[:6], None, None, p[9], need, None) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(ctypes.byref(d), 1e-6, *p[:5], None, None, None, p[9], need, None) == _lib.LORA_ERR_INVALID_ARG
    assert fwd(ctypes.byref(d), 1e-6, *p[:6], None, None, p[9], need - 1, None) == _lib.LORA_ERR_WORKSPACE_TOO_SMALL
    assert bwd(ctypes.byref(d), 1e-6, *p[:6], None, None, p[0], p[7], p[8], p[9], need,
               None) == _lib.LORA_ERR_INVALID_ARG                                                  # dX aliases dY
    bad = lla.GroupDesc(64, 256, (256, 64), 16, 32.0, dtype=lla.LORA_DTYPE_F32).c()
    assert fwd(ctypes.byref(bad), 1e-6, *p[:6], None, None, p[9], need, None) == _lib.LORA_ERR_UNSUPPORTED


def test_w_transposed_flag_checks():
    """LORA_FLAG_W_TRANSPOSED: accepted for bf16 layers and groups, refused for
    the 4-bit and float32 paths and by the tuner; lora_transpose_weight's
    argument checks; the input-gradient GEMM's W^T resource fits 32 bits."""
    L = lib()
    out = ctypes.c_size_t()
    d = lla.Desc(64, 256, 128, 8, 16.0, flags=lla.LORA_FLAG_W_TRANSPOSED).c()
    assert L.lora_linear_workspace_size(ctypes.byref(d), ctypes.byref(out)) == _lib.LORA_OK
    d32 = lla.Desc(64, 256, 128, 8, 16.0, lla.LORA_DTYPE_F32, lla.LORA_FLAG_W_TRANSPOSED).c()
    assert L.lora_linear_workspace_size(ctypes.byref(d32), ctypes.byref(out)) == _lib.LORA_ERR_UNSUPPORTED
    p = [ALIGNED + 0x100 * i for i in range(16)]
    assert L.lora_qlinear_fwd(ctypes.byref(d), *p[:7], None, p[9], 1 << 20, None) == _lib.LORA_ERR_UNSUPPORTED
    assert L.lora_linear_workspace_size(ctypes.byref(lla.Desc(64, 256, 128, 8, 16.0, flags=0x4).c()),
                                        ctypes.byref(out)) == _lib.LORA_ERR_INVALID_ARG
    gd = lla.GroupDesc(64, 256, (256, 64), 16, 32.0, flags=lla.LORA_FLAG_W_TRANSPOSED).c()
    assert L.lora_group_workspace_size(ctypes.byref(gd), ctypes.byref(out)) == _lib.LORA_OK
    cfg = _lib.LoraTunedConfig()
    assert L.lora_tune_linear(ctypes.byref(d), 0, *p[:2], None, None, None, *p[2:11], 1 << 30, None, 3,
                              ctypes.byref(cfg)) == _lib.LORA_ERR_UNSUPPORTED
    assert L.lora_transpose_weight(p[0], 128, 252, p[1], None) == _lib.LORA_ERR_UNSUPPORTED
    assert L.lora_transpose_weight(p[0], 0, 256, p[1], None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_transpose_weight(p[0], 128, 256, p[0], None) == _lib.LORA_ERR_INVALID_ARG
    assert L.lora_transpose_weight(MISALIGNED, 128, 256, p[1], None) == _lib.LORA_ERR_MISALIGNED
    big = lla.Desc(4096, 4096, 14336, 64, 16.0, flags=lla.LORA_FLAG_W_TRANSPOSED)
    ranges = lla.lora_linear_buffer_ranges(big)
    assert ("lora_gemm (dX)", "W^T panel", 256 * 14336 * 2) in ranges
    assert all(b <= 2 ** 31 - 1 for _, _, b in ranges)


# ------------------------------------------------------------ tuning cache (host only)
def test_tuner_cache_file_round_trip(tmp_path):
    """Entries loaded from a cache file are found for their (architecture,
    compute units, shape, weight format) and nowhere else; saving writes them
    back; clearing empties the cache."""
    lla.lora_tuner_clear()
    f = tmp_path / "tune.txt"
    f.write_text("# comment line\n"
                 "gfx950 256 4096 4096 4096 8 0 0 3 2 1 1\n"
                 "gfx950 256 2048 8192 28672 16 1 1 2 4 2 2\n")
    lla.lora_tuner_load(f)
    d = lla.Desc(4096, 4096, 4096, 8, 32.0)
    assert lla.lora_tuner_lookup(d, False, "gfx950", 256) == {"fwd_split": 0, "bwd_split": 3, "rank_div": 2,
                                                              "z_div_fwd": 1, "z_div_bwd": 1}
    assert lla.lora_tuner_lookup(d, True, "gfx950", 256) is None            # the 4-bit layer is another entry
    assert lla.lora_tuner_lookup(d, False, "gfx950", 304) is None            # another compute-unit count
    assert lla.lora_tuner_lookup(lla.Desc(2048, 8192, 28672, 16, 32.0), True, "gfx950", 256)["rank_div"] == 4
    out = tmp_path / "saved.txt"
    lla.lora_tuner_save(out)
    lines = [l for l in out.read_text().splitlines() if not l.startswith("#")]
    assert sorted(lines) == sorted(["gfx950 256 4096 4096 4096 8 0 0 3 2 1 1",
                                    "gfx950 256 2048 8192 28672 16 1 1 2 4 2 2"])
    lla.lora_tuner_clear()
    assert lla.lora_tuner_lookup(d, False, "gfx950", 256) is None


def test_tuner_load_rejects_malformed_files(tmp_path):
    lla.lora_tuner_clear()
    for bad in ("gfx950 256 4096 4096 4096 8 0 0 3 2 1\n",          # a field missing
                "gfx950 256 4096 4096 4096 8 0 5 0 1 1 1\n",         # split mode 5
                "gfx950 256 4096 4096 4096 8 0 0 0 3 1 1\n",         # divisor 3
                "gfx950 0 4096 4096 4096 8 0 0 0 1 1 1\n"):          # no compute units
        f = tmp_path / "bad.txt"
        f.write_text("gfx950 256 64 256 256 8 0 0 0 1 1 1\n" + bad)
        with pytest.raises(lla.LoraError, match="bad.txt:2"):
            lla.lora_tuner_load(f)
        # nothing of a rejected file is merged
        assert lla.lora_tuner_lookup(lla.Desc(64, 256, 256, 8, 32.0), False, "gfx950", 256) is None
    with pytest.raises(lla.LoraError):
        lla.lora_tuner_load(tmp_path / "missing.txt")
