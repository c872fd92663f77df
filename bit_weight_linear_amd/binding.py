"""Thin ctypes binding over libobl's C ABI (include/obl.h).

Argument marshalling only: tensors are passed as device pointers with their
sizes and dtypes, the stream is torch's current HIP stream, and every step of
the computation runs in the library's HIP kernels.  Importing this module
loads ``lib/libobl.so`` and raises ImportError when it is missing; there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libobl.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"libobl.so not built ({_LIB_PATH}); run `python -m bit_weight_linear_amd.build`")

lib = ctypes.CDLL(_LIB_PATH)

# obl_status codes
OBL_OK, OBL_ERR_NULL, OBL_ERR_SHAPE, OBL_ERR_DTYPE, OBL_ERR_ALIGN, OBL_ERR_ALIAS, OBL_ERR_HIP, \
    OBL_ERR_INTERNAL, OBL_ERR_VALUE = range(9)
# obl_dtype codes
OBL_F32, OBL_F16, OBL_BF16, OBL_I8 = range(4)

EXPORTS = ("obl_pack_signs", "obl_linear", "dbf_linear", "obl_transpose_signs", "obl_linear_backward",
           "obl_svid", "obl_layernorm", "obl_linear_layernorm", "obl_status_string", "obl_version")

_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
lib.obl_pack_signs.argtypes = [_vp, _int, _i64, _i64, _vp, _vp]
lib.obl_pack_signs.restype = _int
lib.obl_linear.argtypes = [_vp, _int, _i64, _i64, _vp, _i64, _vp, _vp, _int, _vp, _int, _vp]
lib.obl_linear.restype = _int
lib.dbf_linear.argtypes = [_vp, _int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _int,
                           _vp, _vp, _int, _vp]
lib.dbf_linear.restype = _int
lib.obl_transpose_signs.argtypes = [_vp, _i64, _i64, _vp, _vp]
lib.obl_transpose_signs.restype = _int
lib.obl_linear_backward.argtypes = [_vp, _vp, _int, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _int,
                                    _vp, _int, _vp, _vp, _vp, _vp]
lib.obl_linear_backward.restype = _int
lib.obl_svid.argtypes = [_vp, _int, _i64, _i64, _int, _vp, _vp, _vp, _int, _vp]
lib.obl_svid.restype = _int
_f32 = ctypes.c_float
lib.obl_layernorm.argtypes = [_vp, _int, _i64, _i64, _f32, _vp, _vp, _int, _vp, _int, _vp]
lib.obl_layernorm.restype = _int
lib.obl_linear_layernorm.argtypes = [_vp, _int, _i64, _i64, _vp, _i64, _vp, _vp, _int, _f32, _vp, _vp,
                                     _vp, _vp, _int, _vp]
lib.obl_linear_layernorm.restype = _int
lib.obl_status_string.argtypes = [_int]
lib.obl_status_string.restype = ctypes.c_char_p
lib.obl_version.argtypes = []
lib.obl_version.restype = _int

_DT = {torch.float32: OBL_F32, torch.float16: OBL_F16, torch.bfloat16: OBL_BF16, torch.int8: OBL_I8}


class OblError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {lib.obl_status_string(status).decode()}")


def _check(status: int, call: str):
    if status != OBL_OK:
        raise OblError(status, call)


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    return _DT[dt]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def pack_signs(S: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Pack a [rows, K] sign (or real) matrix into int32 words [rows, K/32] (uint32 bits)."""
    _dev(S, "S")
    rows, K = S.shape
    if out is None:
        out = torch.empty((rows, K // 32), dtype=torch.int32, device=S.device)
    _check(lib.obl_pack_signs(_ptr(S), dtype_code(S.dtype), rows, K, _ptr(out), _stream(S)),
           "obl_pack_signs")
    return out


def linear(X: torch.Tensor, W_packed: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
           out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = ((X ⊙ b) W_sign^T) ⊙ a through ``obl_linear``."""
    for t, n in ((X, "X"), (W_packed, "W_packed"), (a, "a"), (b, "b")):
        _dev(t, n)
    M, K = X.shape
    N = W_packed.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    _check(lib.obl_linear(_ptr(X), dtype_code(X.dtype), M, K, _ptr(W_packed), N, _ptr(a), _ptr(b),
                          dtype_code(a.dtype), _ptr(out), dtype_code(out.dtype), _stream(X)),
           "obl_linear")
    return out


def dbf_linear(X: torch.Tensor, S2_packed: torch.Tensor, S1_packed: torch.Tensor, b: torch.Tensor,
               m: torch.Tensor, a: torch.Tensor, out_dtype: torch.dtype = torch.float32,
               workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Y = ((((X ⊙ b) S2^T) ⊙ m) S1^T) ⊙ a through ``dbf_linear``.

    Returns (Y, workspace); the workspace holds T1 = ((X ⊙ b) S2^T) ⊙ m in fp32.
    """
    for t, n in ((X, "X"), (S2_packed, "S2_packed"), (S1_packed, "S1_packed"), (b, "b"), (m, "m"), (a, "a")):
        _dev(t, n)
    M, K = X.shape
    Kmid = S2_packed.shape[0]
    N = S1_packed.shape[0]
    if workspace is None:
        workspace = torch.empty((M, Kmid), dtype=torch.float32, device=X.device)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    _check(lib.dbf_linear(_ptr(X), dtype_code(X.dtype), M, K, _ptr(S2_packed), Kmid, _ptr(S1_packed), N,
                          _ptr(b), _ptr(m), _ptr(a), dtype_code(a.dtype), _ptr(workspace), _ptr(out),
                          dtype_code(out.dtype), _stream(X)), "dbf_linear")
    return out, workspace


def transpose_signs(P: torch.Tensor, rows: int, K: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed signs of the transposed matrix: [K, rows/32] from [rows, K/32]."""
    _dev(P, "P")
    if out is None:
        out = torch.empty((K, rows // 32), dtype=torch.int32, device=P.device)
    _check(lib.obl_transpose_signs(_ptr(P), rows, K, _ptr(out), _stream(P)), "obl_transpose_signs")
    return out


def linear_backward(dY: torch.Tensor, X: torch.Tensor, W_packed: torch.Tensor, Wt_packed: torch.Tensor,
                    a: torch.Tensor, b: torch.Tensor, dx_dtype: torch.dtype = torch.float32,
                    workspace: Optional[torch.Tensor] = None):
    """(dX, da, db) of Y = ((X ⊙ b) W_sign^T) ⊙ a for the upstream gradient dY,
    through ``obl_linear_backward``.  Returns (dX, da, db, workspace); the
    flat fp32 workspace holds T = (X ⊙ b) W_sign^T [M][N], then U = (dY ⊙ a) W_sign [M][K]."""
    for t, n in ((dY, "dY"), (X, "X"), (W_packed, "W_packed"), (Wt_packed, "Wt_packed"), (a, "a"), (b, "b")):
        _dev(t, n)
    M, K = X.shape
    N = W_packed.shape[0]
    if workspace is None:
        workspace = torch.empty(M * (N + K), dtype=torch.float32, device=X.device)
    dX = torch.empty((M, K), dtype=dx_dtype, device=X.device)
    da = torch.empty(N, dtype=torch.float32, device=X.device)
    db = torch.empty(K, dtype=torch.float32, device=X.device)
    _check(lib.obl_linear_backward(_ptr(dY), _ptr(X), dtype_code(X.dtype), M, K, _ptr(W_packed), _ptr(Wt_packed),
                                   N, _ptr(a), _ptr(b), dtype_code(a.dtype), _ptr(dX), dtype_code(dx_dtype),
                                   _ptr(da), _ptr(db), _ptr(workspace), _stream(X)),
           "obl_linear_backward")
    return dX, da, db, workspace


def svid(W: torch.Tensor, iters: int = 32, scale_dtype: torch.dtype = torch.float16):
    """(packed Sign(W), a, b) with a b^T the rank-1 approximation of |W|, through ``obl_svid``."""
    _dev(W, "W")
    N, K = W.shape
    packed = torch.empty((N, K // 32), dtype=torch.int32, device=W.device)
    a = torch.empty(N, dtype=scale_dtype, device=W.device)
    b = torch.empty(K, dtype=scale_dtype, device=W.device)
    _check(lib.obl_svid(_ptr(W), dtype_code(W.dtype), N, K, iters, _ptr(packed), _ptr(a), _ptr(b),
                        dtype_code(scale_dtype), _stream(W)), "obl_svid")
    return packed, a, b


def layernorm(Y: torch.Tensor, eps: float = 1e-5, gamma: Optional[torch.Tensor] = None,
              beta: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Z = LayerNorm(Y) over rows (optional gamma, beta) through ``obl_layernorm``."""
    _dev(Y, "Y")
    for t, n in ((gamma, "gamma"), (beta, "beta")):
        if t is not None:
            _dev(t, n)
    M, N = Y.shape
    affine = gamma if gamma is not None else beta
    g_dtype = dtype_code(affine.dtype) if affine is not None else OBL_F32
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=Y.device)
    _check(lib.obl_layernorm(_ptr(Y), dtype_code(Y.dtype), M, N, eps, _ptr(gamma), _ptr(beta), g_dtype,
                             _ptr(out), dtype_code(out.dtype), _stream(Y)), "obl_layernorm")
    return out


def linear_layernorm(X: torch.Tensor, W_packed: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                     eps: float = 1e-5, gamma: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.float32, workspace: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None):
    """Z = LayerNorm(((X ⊙ b) W_sign^T) ⊙ a) through ``obl_linear_layernorm``.

    Returns (Z, workspace); the workspace holds the fp32 Y before normalisation."""
    for t, n in ((X, "X"), (W_packed, "W_packed"), (a, "a"), (b, "b")):
        _dev(t, n)
    for t, n in ((gamma, "gamma"), (beta, "beta")):
        if t is not None:
            _dev(t, n)
    M, K = X.shape
    N = W_packed.shape[0]
    if workspace is None:
        workspace = torch.empty((M, N), dtype=torch.float32, device=X.device)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    _check(lib.obl_linear_layernorm(_ptr(X), dtype_code(X.dtype), M, K, _ptr(W_packed), N, _ptr(a), _ptr(b),
                                    dtype_code(a.dtype), eps, _ptr(gamma), _ptr(beta), _ptr(workspace),
                                    _ptr(out), dtype_code(out.dtype), _stream(X)), "obl_linear_layernorm")
    return out, workspace
