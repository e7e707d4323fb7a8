"""ctypes binding of libtpmlp (include/tpmlp.h).

Argument marshalling only: every step of the MLP runs in the library's HIP
kernels.  Functions keep the C names; tensors are torch tensors on the GPU
(bf16 data as ``torch.bfloat16`` or ``torch.uint16``/``torch.int16`` bits,
float32 outputs as ``torch.float32``); sizes come from the tensors' shapes.
A status other than TPMLP_OK raises :class:`TpmlpError`.

If the shared library has not been built, loading fails loudly; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtpmlp.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "tpmlp.h")

STATUS = {
    0: "TPMLP_OK", 1: "TPMLP_ERR_NULL", 2: "TPMLP_ERR_SHAPE", 3: "TPMLP_ERR_ALIGN",
    4: "TPMLP_ERR_WORKSPACE", 5: "TPMLP_ERR_SHARDS", 6: "TPMLP_ERR_HIP",
    7: "TPMLP_ERR_UNSUPPORTED", 8: "TPMLP_ERR_ALIAS", 9: "TPMLP_ERR_NO_FORWARD",
}
KERNEL_COUNT = 13
MAX_SHARDS = 64


class TpmlpError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {STATUS.get(status, status)} ({detail})")


_lib = None

_vp, _sz, _i64, _int = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int
_PP = ctypes.POINTER(ctypes.c_void_p)

_SIGS = {
    "tpmlp_abi_version": ([], _int),
    "tpmlp_status_str": ([_int], ctypes.c_char_p),
    "tpmlp_last_error": ([], ctypes.c_char_p),
    "tpmlp_kernel_name": ([_int], ctypes.c_char_p),
    "tpmlp_fwd_workspace_bytes": ([_i64, _i64, _i64], _sz),
    "tpmlp_bwd_workspace_bytes": ([_i64, _i64, _i64, _int], _sz),
    "tpmlp_tp_workspace_bytes": ([_int, _i64, _i64, _i64], _sz),
    "tpmlp_saved_activation_bytes": ([_i64, _i64, _i64, _int], _sz),
    "tpmlp_recompute_policy": ([_i64, _i64, _i64, _sz], _int),
    "tpmlp_fwd": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_bwd": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_tp_fwd": ([_vp, _PP, _PP, _PP, _PP, _vp, _int, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_tp_bwd": ([_vp, _vp, _PP, _PP, _PP, _PP, _PP, _PP, _vp, _int, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_tp_fwd_full": ([_vp, _vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_tp_bwd_full": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_shard_sum": ([_PP, _int, _vp, _i64, _vp], _int),
    "tpmlp_fwd_noalloc": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp], _int),
    "tpmlp_sp_workspace_bytes": ([_int, _i64, _i64, _i64], _sz),
    "tpmlp_sp_fwd": ([_PP, _PP, _PP, _PP, _PP, _int, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_sp_bwd": ([_PP, _PP, _PP, _PP, _PP, _PP, _PP, _PP, _int, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_fp8_workspace_bytes": ([_int, _i64, _i64, _i64], _sz),
    "tpmlp_fp8_tp_fwd": ([_vp, _PP, _PP, _PP, _vp, _int, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_fp8_tp_bwd": ([_vp, _vp, _PP, _PP, _PP, _PP, _PP, _vp, _int, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    "tpmlp_fp8_quantize": ([_vp, _i64, _i64, _int, _int, _vp, _vp, _vp], _int),
    "tpmlp_timing_begin": ([_int], _int),
    "tpmlp_timing_begin_kinds": ([_int, ctypes.c_uint], _int),
    "tpmlp_timing_end": ([ctypes.POINTER(_int), ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_int)], _int),
    "tpmlp_timing_records": ([ctypes.POINTER(_int), ctypes.POINTER(ctypes.c_double), _int], _int),
    "tpmlp_timing_dispatches": ([ctypes.POINTER(_int), _int], _int),
}


def header_functions() -> list:
    """Names of the functions include/tpmlp.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tpmlp_\w+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first use).  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m tensor_transformer_mlp_03_amd.build` "
                "(hipcc for gfx950). There is no fallback path.")
        try:  # share torch's HIP runtime (same soname) when torch is present
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int, func: str):
    if status != 0:
        raise TpmlpError(status, func, lib().tpmlp_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr_array(items: Optional[Sequence], n: int):
    if items is None:
        return None
    arr = (ctypes.c_void_p * n)()
    for i in range(n):
        arr[i] = _ptr(items[i]) if items[i] is not None else None
    return ctypes.cast(arr, _PP)


def _bf16(t, name):
    import torch
    if t.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError(f"{name} must hold bf16 bits (bfloat16/uint16/int16), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _f32(t, name):
    import torch
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 tensor")
    return t


# --- queries ------------------------------------------------------------------
def tpmlp_abi_version() -> int:
    return lib().tpmlp_abi_version()


def tpmlp_status_str(status: int) -> str:
    return lib().tpmlp_status_str(status).decode()


def tpmlp_kernel_name(kind: int) -> str:
    return lib().tpmlp_kernel_name(kind).decode()


def tpmlp_fwd_workspace_bytes(M: int, H: int, F_i: int) -> int:
    return lib().tpmlp_fwd_workspace_bytes(M, H, F_i)


def tpmlp_bwd_workspace_bytes(M: int, H: int, F_i: int, recompute: bool) -> int:
    return lib().tpmlp_bwd_workspace_bytes(M, H, F_i, int(bool(recompute)))


def tpmlp_tp_workspace_bytes(t: int, M: int, H: int, F_i: int) -> int:
    return lib().tpmlp_tp_workspace_bytes(t, M, H, F_i)


# --- compute ------------------------------------------------------------------
def tpmlp_fwd(X, A_i, B_i, Z_i, P_save, ws, stream=None):
    """Rank i's forward; shapes X[M,H], A_i[H,F_i], B_i[F_i,H], Z_i[M,H] float32."""
    M, H = X.shape
    F = A_i.shape[1]
    _bf16(X, "X"), _bf16(A_i, "A_i"), _bf16(B_i, "B_i"), _f32(Z_i, "Z_i")
    _shape(B_i, (F, H), "B_i"), _shape(Z_i, (M, H), "Z_i")
    if P_save is not None:
        _bf16(P_save, "P_save"), _shape(P_save, (M, F), "P_save")
    st = lib().tpmlp_fwd(_ptr(X), _ptr(A_i), _ptr(B_i), _ptr(Z_i), _ptr(P_save), M, H, F,
                         _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "tpmlp_fwd")


NOALLOC_SCRATCH_BYTES = 64 << 20  # TPMLP_NOALLOC_SCRATCH_BYTES


def tpmlp_fwd_noalloc(X, A_i, B_i, Z_i, P_save, stream=None):
    """tpmlp_fwd with the library's own device scratch array as its workspace (no
    allocation); shapes whose forward workspace exceeds NOALLOC_SCRATCH_BYTES are
    rejected with TPMLP_ERR_WORKSPACE."""
    M, H = X.shape
    F = A_i.shape[1]
    _bf16(X, "X"), _bf16(A_i, "A_i"), _bf16(B_i, "B_i"), _f32(Z_i, "Z_i")
    _shape(B_i, (F, H), "B_i"), _shape(Z_i, (M, H), "Z_i")
    if P_save is not None:
        _bf16(P_save, "P_save"), _shape(P_save, (M, F), "P_save")
    st = lib().tpmlp_fwd_noalloc(_ptr(X), _ptr(A_i), _ptr(B_i), _ptr(Z_i), _ptr(P_save), M, H, F, _stream(stream))
    _check(st, "tpmlp_fwd_noalloc")


def tpmlp_bwd(dZ, X, A_i, B_i, P_saved, dX_i, dA_i, dB_i, ws, stream=None):
    """Rank i's backward; P_saved None recomputes the pre-activation."""
    M, H = X.shape
    F = A_i.shape[1]
    for t, n in ((dZ, "dZ"), (X, "X"), (A_i, "A_i"), (B_i, "B_i")):
        _bf16(t, n)
    for t, n in ((dX_i, "dX_i"), (dA_i, "dA_i"), (dB_i, "dB_i")):
        _f32(t, n)
    for t, n, shp in ((dZ, "dZ", (M, H)), (A_i, "A_i", (H, F)), (B_i, "B_i", (F, H)), (dX_i, "dX_i", (M, H)),
                      (dA_i, "dA_i", (H, F)), (dB_i, "dB_i", (F, H))):
        _shape(t, shp, n)
    if P_saved is not None:
        _bf16(P_saved, "P_saved"), _shape(P_saved, (M, F), "P_saved")
    st = lib().tpmlp_bwd(_ptr(dZ), _ptr(X), _ptr(A_i), _ptr(B_i), _ptr(P_saved), _ptr(dX_i), _ptr(dA_i),
                         _ptr(dB_i), M, H, F, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "tpmlp_bwd")


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _shards(items, t, shape, name, check, nullable=False):
    """Checks a list of t per-shard tensors (entries None allowed if nullable)."""
    if items is None:
        return
    if len(items) != t:
        raise ValueError(f"{name} has {len(items)} entries, expected t = {t}")
    for i, x in enumerate(items):
        if x is None:
            if not nullable:
                raise ValueError(f"{name}[{i}] is None")
            continue
        check(x, f"{name}[{i}]")
        _shape(x, shape, f"{name}[{i}]")


def _whole(A, B, t, H):
    """F_i of the whole weights A[H, t F_i], B[t F_i, H]."""
    if t < 1 or A.shape[1] % t:
        raise ValueError(f"A has {A.shape[1]} columns, not a multiple of t = {t}")
    _shape(A, (H, A.shape[1]), "A")
    _shape(B, (A.shape[1], H), "B")
    return A.shape[1] // t


def tpmlp_tp_fwd(X, A_sh, B_sh, P_sh, Z_sh, Z, ws, stream=None):
    """All t shards' forward, partials summed into Z[M,H] float32."""
    t = len(A_sh)
    M, H = X.shape
    F = A_sh[0].shape[1]
    _bf16(X, "X"), _f32(Z, "Z"), _shape(Z, (M, H), "Z")
    _shards(A_sh, t, (H, F), "A_sh", _bf16)
    _shards(B_sh, t, (F, H), "B_sh", _bf16)
    _shards(P_sh, t, (M, F), "P_sh", _bf16, nullable=True)
    _shards(Z_sh, t, (M, H), "Z_sh", _f32, nullable=True)
    st = lib().tpmlp_tp_fwd(_ptr(X), _ptr_array(A_sh, t), _ptr_array(B_sh, t), _ptr_array(P_sh, t),
                            _ptr_array(Z_sh, t), _ptr(Z), t, M, H, F, _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "tpmlp_tp_fwd")


def tpmlp_tp_bwd(dZ, X, A_sh, B_sh, P_sh, dA_sh, dB_sh, dX_sh, dX, ws, stream=None):
    """All t shards' backward, dX = sum of the shards' partials."""
    t = len(A_sh)
    M, H = X.shape
    F = A_sh[0].shape[1]
    _bf16(dZ, "dZ"), _shape(dZ, (M, H), "dZ"), _bf16(X, "X"), _f32(dX, "dX"), _shape(dX, (M, H), "dX")
    _shards(A_sh, t, (H, F), "A_sh", _bf16)
    _shards(B_sh, t, (F, H), "B_sh", _bf16)
    _shards(P_sh, t, (M, F), "P_sh", _bf16)
    _shards(dA_sh, t, (H, F), "dA_sh", _f32)
    _shards(dB_sh, t, (F, H), "dB_sh", _f32)
    _shards(dX_sh, t, (M, H), "dX_sh", _f32, nullable=True)
    st = lib().tpmlp_tp_bwd(_ptr(dZ), _ptr(X), _ptr_array(A_sh, t), _ptr_array(B_sh, t), _ptr_array(P_sh, t),
                            _ptr_array(dA_sh, t), _ptr_array(dB_sh, t), _ptr_array(dX_sh, t), _ptr(dX), t, M,
                            H, F, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "tpmlp_tp_bwd")


def tpmlp_tp_fwd_full(X, A, B, P, Z, t, ws, stream=None):
    """All t shards' forward over the whole weights A[H, t F_i], B[t F_i, H] (no shard
    copies); P: None or t blocks [M, F_i] of bf16; Z[M,H] float32 the summed output."""
    M, H = X.shape
    F = _whole(A, B, t, H)
    _bf16(X, "X"), _bf16(A, "A"), _bf16(B, "B"), _f32(Z, "Z"), _shape(Z, (M, H), "Z")
    if P is not None:
        _bf16(P, "P")
        if P.numel() != t * M * F:
            raise ValueError(f"P holds {P.numel()} elements, expected t * M * F_i = {t * M * F}")
    st = lib().tpmlp_tp_fwd_full(_ptr(X), _ptr(A), _ptr(B), _ptr(P), _ptr(Z), t, M, H, F, _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "tpmlp_tp_fwd_full")


def tpmlp_tp_bwd_full(dZ, X, A, B, P, dA, dB, dX, t, ws, stream=None):
    """All t shards' backward over the whole weights; dA[H, t F_i] and dB[t F_i, H] are
    the whole float32 weight gradients, dX the sum of the shards' partials."""
    M, H = X.shape
    F = _whole(A, B, t, H)
    for x, n in ((dZ, "dZ"), (X, "X"), (A, "A"), (B, "B")):
        _bf16(x, n)
    _shape(dZ, (M, H), "dZ")
    for x, n, shp in ((dA, "dA", (H, t * F)), (dB, "dB", (t * F, H)), (dX, "dX", (M, H))):
        _f32(x, n), _shape(x, shp, n)
    if P is not None:
        _bf16(P, "P")
        if P.numel() != t * M * F:
            raise ValueError(f"P holds {P.numel()} elements, expected t * M * F_i = {t * M * F}")
    st = lib().tpmlp_tp_bwd_full(_ptr(dZ), _ptr(X), _ptr(A), _ptr(B), _ptr(P), _ptr(dA), _ptr(dB), _ptr(dX), t,
                                 M, H, F, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "tpmlp_tp_bwd_full")


def tpmlp_sp_workspace_bytes(t: int, M: int, H: int, F_i: int) -> int:
    return lib().tpmlp_sp_workspace_bytes(t, M, H, F_i)


def tpmlp_sp_fwd(X_sl, A_sh, B_sh, P_sh, Z_sl, ws, stream=None):
    """Forward at the sequence-parallel boundary: X_sl[r] and Z_sl[r] are rank r's
    token rows [M/t, H] (bf16 in, float32 out); P_sh: None or t tensors [M, F_i]."""
    t = len(A_sh)
    S, H = X_sl[0].shape
    F = A_sh[0].shape[1]
    _shards(X_sl, t, (S, H), "X_sl", _bf16)
    _shards(Z_sl, t, (S, H), "Z_sl", _f32)
    _shards(A_sh, t, (H, F), "A_sh", _bf16)
    _shards(B_sh, t, (F, H), "B_sh", _bf16)
    _shards(P_sh, t, (S * t, F), "P_sh", _bf16, nullable=True)
    st = lib().tpmlp_sp_fwd(_ptr_array(X_sl, t), _ptr_array(A_sh, t), _ptr_array(B_sh, t), _ptr_array(P_sh, t),
                            _ptr_array(Z_sl, t), t, S * t, H, F, _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream))
    _check(st, "tpmlp_sp_fwd")


def tpmlp_sp_bwd(dZ_sl, X_sl, A_sh, B_sh, P_sh, dA_sh, dB_sh, dX_sl, ws, stream=None):
    """Backward at the sequence-parallel boundary; P_sh None recomputes the
    pre-activations."""
    t = len(A_sh)
    S, H = X_sl[0].shape
    F = A_sh[0].shape[1]
    _shards(dZ_sl, t, (S, H), "dZ_sl", _bf16)
    _shards(X_sl, t, (S, H), "X_sl", _bf16)
    _shards(dX_sl, t, (S, H), "dX_sl", _f32)
    _shards(A_sh, t, (H, F), "A_sh", _bf16)
    _shards(B_sh, t, (F, H), "B_sh", _bf16)
    _shards(P_sh, t, (S * t, F), "P_sh", _bf16)
    _shards(dA_sh, t, (H, F), "dA_sh", _f32)
    _shards(dB_sh, t, (F, H), "dB_sh", _f32)
    st = lib().tpmlp_sp_bwd(_ptr_array(dZ_sl, t), _ptr_array(X_sl, t), _ptr_array(A_sh, t), _ptr_array(B_sh, t),
                            _ptr_array(P_sh, t), _ptr_array(dA_sh, t), _ptr_array(dB_sh, t), _ptr_array(dX_sl, t),
                            t, S * t, H, F, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "tpmlp_sp_bwd")


def tpmlp_saved_activation_bytes(M: int, H: int, F: int, recompute: bool) -> int:
    return lib().tpmlp_saved_activation_bytes(M, H, F, int(recompute))


def tpmlp_recompute_policy(M: int, H: int, F: int, budget_bytes: int) -> int:
    """0: keep the pre-activation, 1: recompute it, -1: neither fits the budget."""
    return lib().tpmlp_recompute_policy(M, H, F, budget_bytes)


def tpmlp_shard_sum(parts, out, stream=None):
    """out = parts[0] + ... + parts[t-1] (float32, in order)."""
    t = len(parts)
    _f32(out, "out")
    for i, p in enumerate(parts):
        _f32(p, f"parts[{i}]")
        if p.numel() != out.numel():
            raise ValueError(f"parts[{i}] holds {p.numel()} elements, out {out.numel()}")
    st = lib().tpmlp_shard_sum(_ptr_array(parts, t), t, _ptr(out), out.numel(), _stream(stream))
    _check(st, "tpmlp_shard_sum")


def tpmlp_fp8_workspace_bytes(t: int, M: int, H: int, F_i: int) -> int:
    return lib().tpmlp_fp8_workspace_bytes(t, M, H, F_i)


def tpmlp_fp8_tp_fwd(X, A_sh, B_sh, P_sh, Z, ws, stream=None):
    """The t-shard forward with FP8 operands (per-tensor scaling), Z[M,H] float32."""
    t = len(A_sh)
    M, H = X.shape
    F = A_sh[0].shape[1]
    _bf16(X, "X"), _f32(Z, "Z"), _shape(Z, (M, H), "Z")
    _shards(A_sh, t, (H, F), "A_sh", _bf16)
    _shards(B_sh, t, (F, H), "B_sh", _bf16)
    _shards(P_sh, t, (M, F), "P_sh", _bf16, nullable=True)
    st = lib().tpmlp_fp8_tp_fwd(_ptr(X), _ptr_array(A_sh, t), _ptr_array(B_sh, t), _ptr_array(P_sh, t), _ptr(Z),
                                t, M, H, F, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "tpmlp_fp8_tp_fwd")


def tpmlp_fp8_tp_bwd(dZ, X, A_sh, B_sh, P_sh, dA_sh, dB_sh, dX, ws, stream=None):
    """The t-shard backward with FP8 operands; P_sh None recomputes P_i."""
    t = len(A_sh)
    M, H = X.shape
    F = A_sh[0].shape[1]
    _bf16(dZ, "dZ"), _shape(dZ, (M, H), "dZ"), _bf16(X, "X"), _f32(dX, "dX"), _shape(dX, (M, H), "dX")
    _shards(A_sh, t, (H, F), "A_sh", _bf16)
    _shards(B_sh, t, (F, H), "B_sh", _bf16)
    _shards(P_sh, t, (M, F), "P_sh", _bf16)
    _shards(dA_sh, t, (H, F), "dA_sh", _f32)
    _shards(dB_sh, t, (F, H), "dB_sh", _f32)
    st = lib().tpmlp_fp8_tp_bwd(_ptr(dZ), _ptr(X), _ptr_array(A_sh, t), _ptr_array(B_sh, t), _ptr_array(P_sh, t),
                                _ptr_array(dA_sh, t), _ptr_array(dB_sh, t), _ptr(dX), t, M, H, F, _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "tpmlp_fp8_tp_bwd")


def tpmlp_fp8_quantize(T, fmt: int, transpose: bool, codes, amax, stream=None):
    """FP8 codes of a bf16 tensor T[R,C] (uint8 codes [R,C], or [C,R] transposed) and
    its amax (one float32 element, overwritten)."""
    import torch
    R, C = T.shape
    _bf16(T, "T")
    if codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise TypeError("codes must be a contiguous uint8 tensor")
    _shape(codes, (C, R) if transpose else (R, C), "codes")
    _f32(amax, "amax")
    if amax.numel() != 1:
        raise ValueError("amax must hold one float32")
    st = lib().tpmlp_fp8_quantize(_ptr(T), R, C, int(fmt), 1 if transpose else 0, _ptr(codes), _ptr(amax),
                                  _stream(stream))
    _check(st, "tpmlp_fp8_quantize")


def tpmlp_timing_begin(capacity: int):
    _check(lib().tpmlp_timing_begin(capacity), "tpmlp_timing_begin")


def tpmlp_timing_begin_kinds(capacity: int, kinds):
    """Time only the launches of the named kernel kinds."""
    mask = 0
    for name in kinds:
        mask |= 1 << kernel_kind(name)
    _check(lib().tpmlp_timing_begin_kinds(capacity, mask), "tpmlp_timing_begin_kinds")


def kernel_kind(name: str) -> int:
    for k in range(KERNEL_COUNT):
        if tpmlp_kernel_name(k) == name:
            return k
    raise ValueError(f"no kernel kind named {name!r}")


def tpmlp_timing_end():
    """Returns ({kernel name: (launches, total ms)}, dropped)."""
    counts = (ctypes.c_int * KERNEL_COUNT)()
    total = (ctypes.c_double * KERNEL_COUNT)()
    dropped = ctypes.c_int(0)
    _check(lib().tpmlp_timing_end(counts, total, ctypes.byref(dropped)), "tpmlp_timing_end")
    return {tpmlp_kernel_name(k): (counts[k], total[k]) for k in range(KERNEL_COUNT)}, dropped.value


def tpmlp_timing_records():
    """[(kernel name, ms)] of the last timing window, in launch order."""
    n = lib().tpmlp_timing_records((ctypes.c_int * 1)(), (ctypes.c_double * 1)(), 0)
    kinds = (ctypes.c_int * max(n, 1))()
    ms = (ctypes.c_double * max(n, 1))()
    n = lib().tpmlp_timing_records(kinds, ms, n)
    return [(tpmlp_kernel_name(kinds[i]), ms[i]) for i in range(n)]


def tpmlp_timing_dispatches():
    """Kernel dispatches inside each record of the last timing window (1, or 2
    for a product run as whole-wave tiles plus a split tail)."""
    n = lib().tpmlp_timing_dispatches((ctypes.c_int * 1)(), 0)
    out = (ctypes.c_int * max(n, 1))()
    n = lib().tpmlp_timing_dispatches(out, n)
    return [out[i] for i in range(n)]
