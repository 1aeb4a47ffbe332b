"""Python binding of the C ABI: same names, argument marshalling only.

Each function takes torch tensors (or raw integer device addresses, or None
for optional arguments), passes their addresses and the current HIP stream to
liblora_linear.so, and raises LoraError when the library returns a status
other than LORA_OK.  All arithmetic happens in the library's kernels.
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib
from ._lib import (LORA_DTYPE_BF16, LORA_DTYPE_F32, LORA_FLAG_ACCUM_GRADS, LORA_MAX_MEMBERS,  # noqa: F401
                   LoraBufferRange, LoraGroupDesc, LoraLinearDesc, LoraTunedConfig)


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        self.status = status
        text = lib.lora_status_string(status).decode()
        detail = lib.lora_last_error().decode()
        super().__init__(f"{where}: {text} (status {status}){': ' + detail if detail else ''}")


@dataclasses.dataclass(frozen=True)
class Desc:
    """Problem descriptor (mirrors struct lora_linear_desc)."""
    M: int
    K: int
    N: int
    r: int
    alpha: float
    dtype: int = LORA_DTYPE_BF16
    flags: int = 0

    def c(self) -> LoraLinearDesc:
        return LoraLinearDesc(self.M, self.K, self.N, self.r, float(self.alpha), self.dtype, self.flags)

    @property
    def scale(self) -> float:
        return self.alpha / self.r


@dataclasses.dataclass(frozen=True)
class GroupDesc:
    """Linears sharing one input (mirrors struct lora_group_desc): member m has
    N[m] output columns; W, B, H, dY are stacked by output columns and A, U, V
    by rank rows (m r .. m r + r - 1)."""
    M: int
    K: int
    N: tuple
    r: int
    alpha: float
    dtype: int = LORA_DTYPE_BF16
    flags: int = 0

    def c(self) -> LoraGroupDesc:
        Ns = list(self.N)
        if not 1 <= len(Ns) <= LORA_MAX_MEMBERS:
            raise ValueError(f"a group has 1 .. {LORA_MAX_MEMBERS} members, got {len(Ns)}")
        arr = (ctypes.c_int64 * LORA_MAX_MEMBERS)(*(Ns + [0] * (LORA_MAX_MEMBERS - len(Ns))))
        return LoraGroupDesc(self.M, self.K, self.r, float(self.alpha), self.dtype, self.flags, len(Ns), arr)

    @property
    def N_total(self) -> int:
        return int(sum(self.N))

    @property
    def rank_total(self) -> int:
        return len(self.N) * self.r

    @property
    def scale(self) -> float:
        return self.alpha / self.r


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a tensor, an int address or None, got {type(t)!r}")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous (dense row-major)")
    return t.data_ptr()


_TORCH_DTYPE = {LORA_DTYPE_BF16: torch.bfloat16, LORA_DTYPE_F32: torch.float32}


def _expect(t, name, shape, dtypes):
    """Shape and dtype of a tensor argument (raw integer addresses and None
    pass unchecked)."""
    if t is None or isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor, an int address or None, got {type(t)!r}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")


def _same_gpu(**ts):
    """All tensor arguments on one GPU (checked after their shapes and dtypes)."""
    dev = None
    for name, t in ts.items():
        if not isinstance(t, torch.Tensor):
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name}: tensor on {t.device}, expected a GPU tensor")
        if dev is not None and t.device != dev:
            raise ValueError(f"{name}: tensor on {t.device}, the other operands are on {dev}")
        dev = t.device


def _w_shape(desc, N, K, backward: bool):
    """W [N, K], or W^T [K, N] in a backward call with LORA_FLAG_W_TRANSPOSED."""
    return (K, N) if backward and (desc.flags & _lib.LORA_FLAG_W_TRANSPOSED) else (N, K)


def _check_dense(desc: "Desc", **ts):
    """Operands of a forward or backward call against the descriptor, before
    their addresses go to the library."""
    M, K, N, r = desc.M, desc.K, desc.N, desc.r
    dt = (_TORCH_DTYPE[desc.dtype],) if desc.dtype in _TORCH_DTYPE else ()
    spec = {"X": ((M, K), dt), "W": (_w_shape(desc, N, K, "dY" in ts), dt), "A": ((r, K), dt), "B": ((N, r), dt), "H": ((M, N), dt),
            "dY": ((M, N), dt), "dX": ((M, K), dt), "dA": ((r, K), dt), "dB": ((N, r), dt),
            "U_save": ((M, r), (torch.float32,)), "U_saved": ((M, r), (torch.float32,)),
            "Wq": ((N, K // 2), (torch.uint8,)),
            "absmax": ((N, K // 64), (torch.int16, torch.float16, torch.uint16)),
            "codebook": ((16,), (torch.float32,))}
    for name, t in ts.items():
        _expect(t, name, *spec[name])
    _same_gpu(**ts)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != _lib.LORA_OK:
        raise LoraError(status, where)


def _ws(desc: Desc, ws, device):
    if ws is not None:
        return ws, (ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else None)
    nbytes = lora_linear_workspace_size(desc)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes


def lora_linear_workspace_size(desc: Desc) -> int:
    out = ctypes.c_size_t(0)
    d = desc.c()
    _check(_lib.load().lora_linear_workspace_size(ctypes.byref(d), ctypes.byref(out)), "lora_linear_workspace_size")
    return int(out.value)


def lora_linear_buffer_ranges(desc: Desc, quant: bool = False) -> list:
    """Every buffer resource the kernels may build for this descriptor, as
    (kernel, operand, largest range in bytes) tuples (host only, no HIP call)."""
    d = desc.c()
    n = ctypes.c_int32(0)
    lib = _lib.load()
    _check(lib.lora_linear_buffer_ranges(ctypes.byref(d), int(quant), None, 0, ctypes.byref(n)),
           "lora_linear_buffer_ranges")
    arr = (LoraBufferRange * max(n.value, 1))()
    _check(lib.lora_linear_buffer_ranges(ctypes.byref(d), int(quant), arr, n.value, ctypes.byref(n)),
           "lora_linear_buffer_ranges")
    return [(arr[i].kernel.decode(), arr[i].operand.decode(), int(arr[i].bytes)) for i in range(n.value)]


_timer_ref = None      # keeps the ctypes callback alive while the library holds it


def lora_set_kernel_timer(fn) -> None:
    """fn(kernel: str, stream: int) -> (start_event, stop_event) or None is
    asked before each kernel the library enqueues; the events (hipEvent_t
    handles as ints, created by the caller) are attached to that kernel's
    dispatch and record its start and end.  None removes the timer (see
    include/lora_linear.h)."""
    global _timer_ref
    lib = _lib.load()
    if fn is None:
        lib.lora_set_kernel_timer(_lib.KERNEL_TIMER(), None)
        _timer_ref = None
        return

    def cb(user, kernel, stream, start, stop):
        ev = fn(kernel.decode(), stream or 0)
        if ev is not None:
            start[0], stop[0] = ev[0], ev[1]

    c = _lib.KERNEL_TIMER(cb)
    lib.lora_set_kernel_timer(c, None)
    _timer_ref = c


def lora_linear_fwd(desc: Desc, X, W, A, B, H, U_save=None, ws=None, ws_bytes=None, stream=None):
    """H = X W^T + s (X A^T) B^T (see include/lora_linear.h)."""
    _check_dense(desc, X=X, W=W, A=A, B=B, H=H, U_save=U_save)
    if ws is None:
        ws, ws_bytes = _ws(desc, None, X.device)
    elif ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    d = desc.c()
    st = _lib.load().lora_linear_fwd(ctypes.byref(d), _ptr(X), _ptr(W), _ptr(A), _ptr(B), _ptr(H), _ptr(U_save),
                                     _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "lora_linear_fwd")


def lora_linear_bwd(desc: Desc, dY, X, W, A, B, U_saved, dX, dA, dB, ws=None, ws_bytes=None, stream=None):
    """dX = dY W + s (dY B) A; dA = s (dY B)^T X; dB = s dY^T U (see include/lora_linear.h)."""
    _check_dense(desc, dY=dY, X=X, W=W, A=A, B=B, U_saved=U_saved, dX=dX, dA=dA, dB=dB)
    if ws is None:
        ws, ws_bytes = _ws(desc, None, dY.device)
    elif ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    d = desc.c()
    st = _lib.load().lora_linear_bwd(ctypes.byref(d), _ptr(dY), _ptr(X), _ptr(W), _ptr(A), _ptr(B), _ptr(U_saved),
                                     _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "lora_linear_bwd")


def lora_linear_bwd_noalloc(desc: Desc, dY, X, W, A, B, U_saved, dX, dA, dB, stream=None):
    """lora_linear_bwd with the intermediates in the library's static device
    array instead of a workspace (for callers that cannot allocate)."""
    _check_dense(desc, dY=dY, X=X, W=W, A=A, B=B, U_saved=U_saved, dX=dX, dA=dA, dB=dB)
    d = desc.c()
    st = _lib.load().lora_linear_bwd_noalloc(ctypes.byref(d), _ptr(dY), _ptr(X), _ptr(W), _ptr(A), _ptr(B),
                                             _ptr(U_saved), _ptr(dX), _ptr(dA), _ptr(dB), _stream(stream))
    _check(st, "lora_linear_bwd_noalloc")


def _check_group(g: GroupDesc, **ts):
    M, K, N, R, r = g.M, g.K, g.N_total, g.rank_total, g.r
    dt = (_TORCH_DTYPE[g.dtype],) if g.dtype in _TORCH_DTYPE else ()
    spec = {"X": ((M, K), dt), "W": (_w_shape(g, N, K, "dY" in ts), dt), "A": ((R, K), dt), "B": ((N, r), dt), "H": ((M, N), dt),
            "dY": ((M, N), dt), "dX": ((M, K), dt), "dA": ((R, K), dt), "dB": ((N, r), dt),
            "U_save": ((M, R), (torch.float32,)), "U_saved": ((M, R), (torch.float32,))}
    for name, t in ts.items():
        _expect(t, name, *spec[name])
    _same_gpu(**ts)


def lora_group_workspace_size(desc: GroupDesc) -> int:
    out = ctypes.c_size_t(0)
    d = desc.c()
    _check(_lib.load().lora_group_workspace_size(ctypes.byref(d), ctypes.byref(out)), "lora_group_workspace_size")
    return int(out.value)


def _group_ws(desc, ws, ws_bytes, device):
    if ws is None:
        nbytes = lora_group_workspace_size(desc)
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    return ws, ws_bytes


def lora_group_fwd(desc: GroupDesc, X, W, A, B, H, U_save=None, ws=None, ws_bytes=None, stream=None):
    """H_m = X W_m^T + s (X A_m^T) B_m^T for every member (stacked layout, see include/lora_linear.h)."""
    _check_group(desc, X=X, W=W, A=A, B=B, H=H, U_save=U_save)
    ws, ws_bytes = _group_ws(desc, ws, ws_bytes, X.device)
    d = desc.c()
    st = _lib.load().lora_group_fwd(ctypes.byref(d), _ptr(X), _ptr(W), _ptr(A), _ptr(B), _ptr(H), _ptr(U_save),
                                    _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "lora_group_fwd")


def lora_group_bwd(desc: GroupDesc, dY, X, W, A, B, U_saved, dX, dA, dB, ws=None, ws_bytes=None, stream=None):
    """dX = sum_m (dY_m W_m + s V_m A_m); dA_m, dB_m per member (stacked layout)."""
    _check_group(desc, dY=dY, X=X, W=W, A=A, B=B, U_saved=U_saved, dX=dX, dA=dA, dB=dB)
    ws, ws_bytes = _group_ws(desc, ws, ws_bytes, dY.device)
    d = desc.c()
    st = _lib.load().lora_group_bwd(ctypes.byref(d), _ptr(dY), _ptr(X), _ptr(W), _ptr(A), _ptr(B), _ptr(U_saved),
                                    _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "lora_group_bwd")


def _check_norm(desc: Desc, **ts):
    M, K, N, r = desc.M, desc.K, desc.N, desc.r
    bf = (torch.bfloat16,)
    spec = {"X": ((M, K), bf), "g": ((K,), bf), "W": ((N, K), bf), "W_g": (_w_shape(desc, N, K, "dY" in ts), bf),
            "A": ((r, K), bf),
            "B": ((N, r), bf), "H": ((M, N), bf), "dY": ((M, N), bf), "dX": ((M, K), bf), "dA": ((r, K), bf),
            "dB": ((N, r), bf), "U_save": ((M, r), (torch.float32,)), "U_saved": ((M, r), (torch.float32,)),
            "inv_rms_save": ((M,), (torch.float32,)), "inv_rms_saved": ((M,), (torch.float32,))}
    for name, t in ts.items():
        _expect(t, name, *spec[name])
    _same_gpu(**ts)


def lora_norm_linear_workspace_size(desc: Desc) -> int:
    out = ctypes.c_size_t(0)
    d = desc.c()
    _check(_lib.load().lora_norm_linear_workspace_size(ctypes.byref(d), ctypes.byref(out)),
           "lora_norm_linear_workspace_size")
    return int(out.value)


def lora_transpose_weight(W, Wt, stream=None):
    """Wt = W^T (bf16 [N, K] -> [K, N]): the frozen weight's copy for backward
    calls with LORA_FLAG_W_TRANSPOSED."""
    N, K = W.shape
    _expect(W, "W", (N, K), (torch.bfloat16,))
    _expect(Wt, "Wt", (K, N), (torch.bfloat16,))
    _same_gpu(W=W, Wt=Wt)
    _check(_lib.load().lora_transpose_weight(_ptr(W), N, K, _ptr(Wt), _stream(stream)), "lora_transpose_weight")


def lora_fold_norm_weight(W, g, W_out, stream=None):
    """W_out = bf16(W diag(g)): the frozen RMSNorm weight folded into the frozen
    linear weight once (W_out may be W)."""
    N, K = W.shape
    for name, t, shape in (("W", W, (N, K)), ("g", g, (K,)), ("W_out", W_out, (N, K))):
        _expect(t, name, shape, (torch.bfloat16,))
    _same_gpu(W=W, g=g, W_out=W_out)
    st = _lib.load().lora_fold_norm_weight(_ptr(W), _ptr(g), N, K, _ptr(W_out), _stream(stream))
    _check(st, "lora_fold_norm_weight")


def _norm_ws(desc, ws, ws_bytes, device):
    if ws is None:
        nbytes = lora_norm_linear_workspace_size(desc)
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    return ws, ws_bytes


def lora_norm_linear_fwd(desc: Desc, eps: float, X, g, W_g, A, B, H, U_save=None, inv_rms_save=None, ws=None,
                         ws_bytes=None, stream=None):
    """H = Xn W^T + s (Xn A^T) B^T with Xn = RMSNorm(X) g, from the raw X and
    the folded W_g (see include/lora_linear.h)."""
    _check_norm(desc, X=X, g=g, W_g=W_g, A=A, B=B, H=H, U_save=U_save, inv_rms_save=inv_rms_save)
    ws, ws_bytes = _norm_ws(desc, ws, ws_bytes, X.device)
    d = desc.c()
    st = _lib.load().lora_norm_linear_fwd(ctypes.byref(d), float(eps), _ptr(X), _ptr(g), _ptr(W_g), _ptr(A),
                                          _ptr(B), _ptr(H), _ptr(U_save), _ptr(inv_rms_save), _ptr(ws), ws_bytes,
                                          _stream(stream))
    _check(st, "lora_norm_linear_fwd")


def lora_norm_linear_bwd(desc: Desc, eps: float, dY, X, g, W_g, A, B, U_saved, inv_rms_saved, dX, dA, dB,
                         ws=None, ws_bytes=None, stream=None):
    """dX through the norm to the raw X; dA = s (dY B)^T Xn; dB = s dY^T U."""
    _check_norm(desc, dY=dY, X=X, g=g, W_g=W_g, A=A, B=B, U_saved=U_saved, inv_rms_saved=inv_rms_saved, dX=dX,
                dA=dA, dB=dB)
    ws, ws_bytes = _norm_ws(desc, ws, ws_bytes, dY.device)
    d = desc.c()
    st = _lib.load().lora_norm_linear_bwd(ctypes.byref(d), float(eps), _ptr(dY), _ptr(X), _ptr(g), _ptr(W_g),
                                          _ptr(A), _ptr(B), _ptr(U_saved), _ptr(inv_rms_saved), _ptr(dX), _ptr(dA),
                                          _ptr(dB), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "lora_norm_linear_bwd")


def _check_norm_group(gd: GroupDesc, **ts):
    M, K, N, R, r = gd.M, gd.K, gd.N_total, gd.rank_total, gd.r
    bf = (torch.bfloat16,)
    spec = {"X": ((M, K), bf), "g": ((K,), bf), "W_g": (_w_shape(gd, N, K, "dY" in ts), bf), "A": ((R, K), bf),
            "B": ((N, r), bf),
            "H": ((M, N), bf), "dY": ((M, N), bf), "dX": ((M, K), bf), "dA": ((R, K), bf), "dB": ((N, r), bf),
            "U_save": ((M, R), (torch.float32,)), "U_saved": ((M, R), (torch.float32,)),
            "inv_rms_save": ((M,), (torch.float32,)), "inv_rms_saved": ((M,), (torch.float32,))}
    for name, t in ts.items():
        _expect(t, name, *spec[name])
    _same_gpu(**ts)


def lora_norm_group_workspace_size(desc: GroupDesc) -> int:
    out = ctypes.c_size_t(0)
    d = desc.c()
    _check(_lib.load().lora_norm_group_workspace_size(ctypes.byref(d), ctypes.byref(out)),
           "lora_norm_group_workspace_size")
    return int(out.value)


def lora_norm_group_fwd(desc: GroupDesc, eps: float, X, g, W_g, A, B, H, U_save=None, inv_rms_save=None, ws=None,
                        ws_bytes=None, stream=None):
    """Every member of the group behind one RMSNorm of X (stacked layout)."""
    _check_norm_group(desc, X=X, g=g, W_g=W_g, A=A, B=B, H=H, U_save=U_save, inv_rms_save=inv_rms_save)
    if ws is None:
        ws_bytes = lora_norm_group_workspace_size(desc)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=X.device)
    elif ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    d = desc.c()
    st = _lib.load().lora_norm_group_fwd(ctypes.byref(d), float(eps), _ptr(X), _ptr(g), _ptr(W_g), _ptr(A), _ptr(B),
                                         _ptr(H), _ptr(U_save), _ptr(inv_rms_save), _ptr(ws), ws_bytes,
                                         _stream(stream))
    _check(st, "lora_norm_group_fwd")


def lora_norm_group_bwd(desc: GroupDesc, eps: float, dY, X, g, W_g, A, B, U_saved, inv_rms_saved, dX, dA, dB,
                        ws=None, ws_bytes=None, stream=None):
    """dX through the norm of the summed members; dA, dB per member."""
    _check_norm_group(desc, dY=dY, X=X, g=g, W_g=W_g, A=A, B=B, U_saved=U_saved, inv_rms_saved=inv_rms_saved,
                      dX=dX, dA=dA, dB=dB)
    if ws is None:
        ws_bytes = lora_norm_group_workspace_size(desc)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dY.device)
    elif ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    d = desc.c()
    st = _lib.load().lora_norm_group_bwd(ctypes.byref(d), float(eps), _ptr(dY), _ptr(X), _ptr(g), _ptr(W_g),
                                         _ptr(A), _ptr(B), _ptr(U_saved), _ptr(inv_rms_saved), _ptr(dX), _ptr(dA),
                                         _ptr(dB), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "lora_norm_group_bwd")


_TUNED_FIELDS = ("fwd_split", "bwd_split", "rank_div", "z_div_fwd", "z_div_bwd", "fwd_us", "bwd_us",
                 "default_fwd_us", "default_bwd_us")


def _tuned_dict(c: LoraTunedConfig) -> dict:
    return {k: (round(getattr(c, k), 2) if k.endswith("_us") else int(getattr(c, k))) for k in _TUNED_FIELDS}


def lora_tune_linear(desc: Desc, X, A, B, H, U, dY, dX, dA, dB, W=None, Wq=None, absmax=None, codebook=None,
                     ws=None, ws_bytes=None, stream=None, reps: int = 5) -> dict:
    """Probe the launch parameters of this layer shape on the current device
    (forward and backward, each candidate timed reps times), cache the fastest
    and return it with the median times (see include/lora_linear.h).  With W
    the plain layer is tuned, with Wq, absmax, codebook the 4-bit one."""
    quant = W is None
    _check_dense(desc, X=X, A=A, B=B, H=H, U_save=U, dY=dY, dX=dX, dA=dA, dB=dB,
                 **({"Wq": Wq, "absmax": absmax, "codebook": codebook} if quant else {"W": W}))
    if ws is None:
        ws, ws_bytes = _ws(desc, None, X.device)
    elif ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    d = desc.c()
    out = LoraTunedConfig()
    st = _lib.load().lora_tune_linear(ctypes.byref(d), int(quant), _ptr(X), _ptr(W), _ptr(Wq), _ptr(absmax),
                                      _ptr(codebook), _ptr(A), _ptr(B), _ptr(H), _ptr(U), _ptr(dY), _ptr(dX),
                                      _ptr(dA), _ptr(dB), _ptr(ws), ws_bytes, _stream(stream), int(reps),
                                      ctypes.byref(out))
    _check(st, "lora_tune_linear")
    return _tuned_dict(out)


def lora_tuner_lookup(desc: Desc, quant: bool = False, arch: str | None = None, cus: int = 0):
    """The cached choice for this descriptor (on the named architecture and
    compute-unit count, or the current device), or None."""
    d = desc.c()
    out = LoraTunedConfig()
    found = ctypes.c_int32(0)
    st = _lib.load().lora_tuner_lookup(arch.encode() if arch else None, int(cus), ctypes.byref(d), int(quant),
                                       ctypes.byref(out), ctypes.byref(found))
    _check(st, "lora_tuner_lookup")
    if not found.value:
        return None
    return {k: v for k, v in _tuned_dict(out).items() if not k.endswith("_us")}


def lora_tuner_save(path: str) -> None:
    _check(_lib.load().lora_tuner_save(str(path).encode()), "lora_tuner_save")


def lora_tuner_load(path: str) -> None:
    _check(_lib.load().lora_tuner_load(str(path).encode()), "lora_tuner_load")


def lora_tuner_clear() -> None:
    _lib.load().lora_tuner_clear()


def lora_qlinear_fwd(desc: Desc, X, Wq, absmax, codebook, A, B, H, U_save=None, ws=None, ws_bytes=None,
                     stream=None):
    """Forward with the frozen weight in the 4-bit format (codes, fp16 absmax, codebook)."""
    _check_dense(desc, X=X, Wq=Wq, absmax=absmax, codebook=codebook, A=A, B=B, H=H, U_save=U_save)
    if ws is None:
        ws, ws_bytes = _ws(desc, None, X.device)
    elif ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    d = desc.c()
    st = _lib.load().lora_qlinear_fwd(ctypes.byref(d), _ptr(X), _ptr(Wq), _ptr(absmax), _ptr(codebook), _ptr(A),
                                      _ptr(B), _ptr(H), _ptr(U_save), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "lora_qlinear_fwd")


def lora_qlinear_bwd(desc: Desc, dY, X, Wq, absmax, codebook, A, B, U_saved, dX, dA, dB, ws=None, ws_bytes=None,
                     stream=None):
    """Backward with the frozen weight in the 4-bit format."""
    _check_dense(desc, dY=dY, X=X, Wq=Wq, absmax=absmax, codebook=codebook, A=A, B=B,
                 U_saved=U_saved, dX=dX, dA=dA, dB=dB)
    if ws is None:
        ws, ws_bytes = _ws(desc, None, dY.device)
    elif ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    d = desc.c()
    st = _lib.load().lora_qlinear_bwd(ctypes.byref(d), _ptr(dY), _ptr(X), _ptr(Wq), _ptr(absmax), _ptr(codebook),
                                      _ptr(A), _ptr(B), _ptr(U_saved), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                      ws_bytes, _stream(stream))
    _check(st, "lora_qlinear_bwd")


def lora_dequant4(Wq, absmax, codebook, N: int, K: int, out_dtype: int, W_out, stream=None):
    """Dense W_out [N, K] from the 4-bit format."""
    _expect(Wq, "Wq", (N, K // 2), (torch.uint8,))
    _expect(absmax, "absmax", (N, K // 64), (torch.int16, torch.float16, torch.uint16))
    _expect(codebook, "codebook", (16,), (torch.float32,))
    _expect(W_out, "W_out", (N, K), (_TORCH_DTYPE.get(out_dtype, torch.bfloat16),))
    _same_gpu(Wq=Wq, absmax=absmax, codebook=codebook, W_out=W_out)
    st = _lib.load().lora_dequant4(_ptr(Wq), _ptr(absmax), _ptr(codebook), N, K, out_dtype, _ptr(W_out),
                                   _stream(stream))
    _check(st, "lora_dequant4")


def lora_merge(desc: Desc, W, A, B, W_out, sign: int = 1, stream=None):
    """W_out = W + sign * s * B A (sign +1 merge, -1 unmerge); W_out may be W (in place)."""
    dt = (_TORCH_DTYPE[desc.dtype],) if desc.dtype in _TORCH_DTYPE else ()
    _expect(W, "W", (desc.N, desc.K), dt)
    _expect(A, "A", (desc.r, desc.K), dt)
    _expect(B, "B", (desc.N, desc.r), dt)
    _expect(W_out, "W_out", (desc.N, desc.K), dt)
    _same_gpu(W=W, A=A, B=B, W_out=W_out)
    d = desc.c()
    st = _lib.load().lora_merge(ctypes.byref(d), _ptr(W), _ptr(A), _ptr(B), _ptr(W_out), int(sign), _stream(stream))
    _check(st, "lora_merge")
