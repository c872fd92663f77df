"""Thin ctypes binding over libobl's C ABI (include/obl.h).

Argument marshalling only: tensors are passed as device pointers with their
sizes and dtypes, the stream is torch's current HIP stream, and every step of
the computation runs in the library's HIP kernels.  Importing this module
loads ``lib/libobl.so`` and raises ImportError when it is missing; there is no
fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libobl.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"libobl.so not built ({_LIB_PATH}); run `python -m bit_weight_linear_amd.build`")

lib = ctypes.CDLL(_LIB_PATH)

# obl_status codes
OBL_OK, OBL_ERR_NULL, OBL_ERR_SHAPE, OBL_ERR_DTYPE, OBL_ERR_ALIGN, OBL_ERR_ALIAS, OBL_ERR_HIP, \
    OBL_ERR_INTERNAL, OBL_ERR_VALUE, OBL_ERR_CAPTURE, OBL_ERR_SCRATCH = range(11)
# obl_dtype codes
OBL_F32, OBL_F16, OBL_BF16, OBL_I8 = range(4)

EXPORTS = ("obl_pack_signs", "obl_linear", "dbf_linear", "dbf_linear_noalloc", "obl_transpose_signs",
           "obl_linear_backward", "obl_svid", "obl_layernorm", "obl_linear_layernorm", "obl_status_string",
           "obl_version")

_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
lib.obl_pack_signs.argtypes = [_vp, _int, _i64, _i64, _vp, _vp]
lib.obl_pack_signs.restype = _int
lib.obl_linear.argtypes = [_vp, _int, _i64, _i64, _vp, _i64, _vp, _vp, _int, _vp, _int, _vp]
lib.obl_linear.restype = _int
lib.dbf_linear.argtypes = [_vp, _int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _int,
                           _vp, _vp, _int, _vp]
lib.dbf_linear.restype = _int
lib.dbf_linear_noalloc.argtypes = lib.dbf_linear.argtypes
lib.dbf_linear_noalloc.restype = _int
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
# Internal export used only by the test suite (not in obl.h): forces a path and
# kernel for the calling thread; see forced_kernels below.
lib.obl_internal_force_kernels.argtypes = [_int, _int, _int, _int]
lib.obl_internal_force_kernels.restype = None
# Internal exports used only by the benchmark (not in obl.h): obl_linear with a
# span record of the GEMV launch, and the measurement kernels of peaks.hip.
lib.obl_internal_linear_span.argtypes = [_vp, _int, _i64, _i64, _vp, _i64, _vp, _vp, _int, _vp, _int, _vp, _vp]
lib.obl_internal_linear_span.restype = _int
lib.obl_internal_wallclock_khz.argtypes = []
lib.obl_internal_wallclock_khz.restype = _int
lib.obl_internal_peak_read.argtypes = [_vp, _i64, _vp, _vp]
lib.obl_internal_peak_read.restype = _int
lib.obl_internal_peak_mfma.argtypes = [_i64, _vp, ctypes.POINTER(ctypes.c_double), _vp]
lib.obl_internal_peak_mfma.restype = _int

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
    """A contiguous tensor on the current HIP device (the library launches there)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t: torch.Tensor, name: str, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _numel(t: torch.Tensor, name: str, n: int):
    if t.dim() != 1 or t.numel() != n:
        raise ValueError(f"{name} must be a vector of {n} elements, got shape {tuple(t.shape)}")


def _dtype(t: torch.Tensor, name: str, allowed):
    if t.dtype not in allowed:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in allowed]}")


_WORD = (torch.int32,) + ((torch.uint32,) if hasattr(torch, "uint32") else ())
_XDT = (torch.float32, torch.bfloat16)
_SDT = (torch.float32, torch.float16)
_YDT = (torch.float32, torch.bfloat16)


def _packed(t: torch.Tensor, name: str, rows: int, K: int):
    """Packed sign words [rows][K/32]."""
    _dev(t, name)
    _dtype(t, name, _WORD)
    if K % 32 != 0:
        raise ValueError(f"the contraction length {K} of {name} is not a multiple of 32")
    _shape(t, name, (rows, K // 32))


def _mat(t: torch.Tensor, name: str):
    _dev(t, name)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape


def _scales(name_vec, n_dtype):
    """Scale vectors: each (tensor, name, length); all of one dtype (f32 or f16)."""
    first = None
    for t, n, ln in name_vec:
        _dev(t, n)
        _numel(t, n, ln)
        _dtype(t, n, _SDT)
        if first is None:
            first = t
        elif t.dtype != first.dtype:
            raise ValueError(f"{n} has dtype {t.dtype}, but the other scale vectors are {first.dtype}")
    return first.dtype


def _out(t: Optional[torch.Tensor], name: str, shape, dtypes, default_dtype, device):
    if t is None:
        if default_dtype not in dtypes:
            raise ValueError(f"{name} dtype {default_dtype} not supported")
        return torch.empty(shape, dtype=default_dtype, device=device)
    _dev(t, name)
    _dtype(t, name, dtypes)
    _shape(t, name, shape)
    return t


_PATHS = {None: 0, "auto": 0, "lut": 1, "decode": 2, "gemm": 3}
_GEMMS = {None: 0, "auto": 0, "v1": 1, "v2": 2, "w1": 11, "w2": 12, "w4": 14, "w7": 17}
_DECODES = {None: 0, "auto": 0, "split": 1, "wk1": 11, "wk2": 12, "wk4": 14}
_PAIRS = {None: 0, "auto": 0, "off": 1}


_forced = threading.local()


def _forced_state():
    return getattr(_forced, "state", {"path": None, "gemm": None, "decode": None, "pair": None})


def _apply_forced(state):
    _forced.state = dict(state)
    lib.obl_internal_force_kernels(_PATHS[state["path"]], _GEMMS[state["gemm"]], _DECODES[state["decode"]],
                                   _PAIRS[state["pair"]])


@contextlib.contextmanager
def forced_kernels(path: Optional[str] = None, gemm: Optional[str] = None, decode: Optional[str] = None,
                   pair: Optional[str] = None):
    """Test-suite hook: force a path ("lut" | "decode" | "gemm"), a prefill kernel or tile ("v1", "v2",
    "w1", "w2", "w4", "w7"), a decode kernel ("split", "wk1", "wk2", "wk4") and whether the backward
    may run its two contractions as one launch ("off": two launches) for this thread's calls inside the
    block (nested blocks combine; arguments left None keep the enclosing choice), through an internal
    export that obl.h does not declare.  Nothing else reaches it: ordinary calls always run the kernel
    their arguments select."""
    old = _forced_state()
    new = dict(old)
    for k, v in (("path", path), ("gemm", gemm), ("decode", decode), ("pair", pair)):
        if v is not None:
            new[k] = v
    _apply_forced(new)
    try:
        yield
    finally:
        _apply_forced(old)


def pack_signs(S: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Pack a [rows, K] sign (or real) matrix into int32 words [rows, K/32] (uint32 bits)."""
    rows, K = _mat(S, "S")
    _dtype(S, "S", tuple(_DT))
    if K % 32 != 0:
        raise ValueError(f"K = {K} is not a multiple of 32")
    if out is None:
        out = torch.empty((rows, K // 32), dtype=torch.int32, device=S.device)
    _packed(out, "out", rows, K)
    _check(lib.obl_pack_signs(_ptr(S), dtype_code(S.dtype), rows, K, _ptr(out), _stream(S)),
           "obl_pack_signs")
    return out


def linear(X: torch.Tensor, W_packed: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
           out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = ((X ⊙ b) W_sign^T) ⊙ a through ``obl_linear``."""
    M, K = _mat(X, "X")
    _dtype(X, "X", _XDT)
    N = _mat(W_packed, "W_packed")[0]
    _packed(W_packed, "W_packed", N, K)
    sdt = _scales([(a, "a", N), (b, "b", K)], None)
    out = _out(out, "out", (M, N), _YDT, out_dtype, X.device)
    _check(lib.obl_linear(_ptr(X), dtype_code(X.dtype), M, K, _ptr(W_packed), N, _ptr(a), _ptr(b),
                          dtype_code(sdt), _ptr(out), dtype_code(out.dtype), _stream(X)),
           "obl_linear")
    return out


def _dbf(fn, name, X, S2_packed, S1_packed, b, m, a, out_dtype, workspace, out):
    M, K = _mat(X, "X")
    _dtype(X, "X", _XDT)
    Kmid = _mat(S2_packed, "S2_packed")[0]
    _packed(S2_packed, "S2_packed", Kmid, K)
    N = _mat(S1_packed, "S1_packed")[0]
    _packed(S1_packed, "S1_packed", N, Kmid)
    sdt = _scales([(b, "b", K), (m, "m", Kmid), (a, "a", N)], None)
    workspace = _out(workspace, "workspace", (M, Kmid), (torch.float32,), torch.float32, X.device)
    out = _out(out, "out", (M, N), _YDT, out_dtype, X.device)
    _check(fn(_ptr(X), dtype_code(X.dtype), M, K, _ptr(S2_packed), Kmid, _ptr(S1_packed), N,
              _ptr(b), _ptr(m), _ptr(a), dtype_code(sdt), _ptr(workspace), _ptr(out),
              dtype_code(out.dtype), _stream(X)), name)
    return out, workspace


def dbf_linear(X: torch.Tensor, S2_packed: torch.Tensor, S1_packed: torch.Tensor, b: torch.Tensor,
               m: torch.Tensor, a: torch.Tensor, out_dtype: torch.dtype = torch.float32,
               workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Y = ((((X ⊙ b) S2^T) ⊙ m) S1^T) ⊙ a through ``dbf_linear``.

    Returns (Y, workspace); the workspace holds T1 = ((X ⊙ b) S2^T) ⊙ m in fp32.
    """
    return _dbf(lib.dbf_linear, "dbf_linear", X, S2_packed, S1_packed, b, m, a, out_dtype, workspace, out)


def dbf_linear_noalloc(X: torch.Tensor, S2_packed: torch.Tensor, S1_packed: torch.Tensor, b: torch.Tensor,
                       m: torch.Tensor, a: torch.Tensor, workspace: torch.Tensor, out: torch.Tensor):
    """``dbf_linear_noalloc``: dbf_linear whose library scratch is a fixed device array (no device
    allocation by the library).  The caller passes the workspace and the output."""
    if workspace is None or out is None:
        raise ValueError("dbf_linear_noalloc takes a caller-allocated workspace and out")
    return _dbf(lib.dbf_linear_noalloc, "dbf_linear_noalloc", X, S2_packed, S1_packed, b, m, a, out.dtype,
                workspace, out)


def transpose_signs(P: torch.Tensor, rows: int, K: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed signs of the transposed matrix: [K, rows/32] from [rows, K/32]."""
    _packed(P, "P", rows, K)
    if rows % 32 != 0:
        raise ValueError(f"rows = {rows} is not a multiple of 32")
    if out is None:
        out = torch.empty((K, rows // 32), dtype=torch.int32, device=P.device)
    _packed(out, "out", K, rows)
    _check(lib.obl_transpose_signs(_ptr(P), rows, K, _ptr(out), _stream(P)), "obl_transpose_signs")
    return out


def linear_backward(dY: torch.Tensor, X: torch.Tensor, W_packed: torch.Tensor, Wt_packed: torch.Tensor,
                    a: torch.Tensor, b: torch.Tensor, dx_dtype: torch.dtype = torch.float32,
                    workspace: Optional[torch.Tensor] = None):
    """(dX, da, db) of Y = ((X ⊙ b) W_sign^T) ⊙ a for the upstream gradient dY,
    through ``obl_linear_backward``.  Returns (dX, da, db, workspace); the
    flat fp32 workspace holds T = (X ⊙ b) W_sign^T [M][N], then U = (dY ⊙ a) W_sign [M][K]."""
    M, K = _mat(X, "X")
    _dtype(X, "X", _XDT)
    N = _mat(W_packed, "W_packed")[0]
    _packed(W_packed, "W_packed", N, K)
    _packed(Wt_packed, "Wt_packed", K, N)
    _mat(dY, "dY")
    _shape(dY, "dY", (M, N))
    if dY.dtype != X.dtype:
        raise ValueError(f"dY has dtype {dY.dtype}, X has {X.dtype}: they must match")
    sdt = _scales([(a, "a", N), (b, "b", K)], None)
    if workspace is None:
        workspace = torch.empty(M * (N + K), dtype=torch.float32, device=X.device)
    _dev(workspace, "workspace")
    _dtype(workspace, "workspace", (torch.float32,))
    if workspace.numel() < M * (N + K):
        raise ValueError(f"workspace holds {workspace.numel()} floats, the call needs M (N + K) = {M * (N + K)}")
    dX = _out(None, "dX", (M, K), _YDT, dx_dtype, X.device)
    da = torch.empty(N, dtype=torch.float32, device=X.device)
    db = torch.empty(K, dtype=torch.float32, device=X.device)
    _check(lib.obl_linear_backward(_ptr(dY), _ptr(X), dtype_code(X.dtype), M, K, _ptr(W_packed), _ptr(Wt_packed),
                                   N, _ptr(a), _ptr(b), dtype_code(sdt), _ptr(dX), dtype_code(dx_dtype),
                                   _ptr(da), _ptr(db), _ptr(workspace), _stream(X)),
           "obl_linear_backward")
    return dX, da, db, workspace


def svid(W: torch.Tensor, iters: int = 32, scale_dtype: torch.dtype = torch.float16):
    """(packed Sign(W), a, b) with a b^T the rank-1 approximation of |W|, through ``obl_svid``."""
    N, K = _mat(W, "W")
    _dtype(W, "W", (torch.float32, torch.float16, torch.bfloat16))
    if scale_dtype not in _SDT:
        raise ValueError(f"scale_dtype {scale_dtype} not supported")
    if K % 32 != 0:
        raise ValueError(f"K = {K} is not a multiple of 32")
    packed = torch.empty((N, K // 32), dtype=torch.int32, device=W.device)
    a = torch.empty(N, dtype=scale_dtype, device=W.device)
    b = torch.empty(K, dtype=scale_dtype, device=W.device)
    _check(lib.obl_svid(_ptr(W), dtype_code(W.dtype), N, K, iters, _ptr(packed), _ptr(a), _ptr(b),
                        dtype_code(scale_dtype), _stream(W)), "obl_svid")
    return packed, a, b


def _affine(gamma, beta, N):
    vecs = [(t, n, N) for t, n in ((gamma, "gamma"), (beta, "beta")) if t is not None]
    return _scales(vecs, None) if vecs else None


def layernorm(Y: torch.Tensor, eps: float = 1e-5, gamma: Optional[torch.Tensor] = None,
              beta: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Z = LayerNorm(Y) over rows (optional gamma, beta) through ``obl_layernorm``."""
    M, N = _mat(Y, "Y")
    _dtype(Y, "Y", _YDT)
    gdt = _affine(gamma, beta, N)
    out = _out(out, "out", (M, N), _YDT, out_dtype, Y.device)
    _check(lib.obl_layernorm(_ptr(Y), dtype_code(Y.dtype), M, N, eps, _ptr(gamma), _ptr(beta),
                             dtype_code(gdt) if gdt is not None else OBL_F32,
                             _ptr(out), dtype_code(out.dtype), _stream(Y)), "obl_layernorm")
    return out


def linear_layernorm(X: torch.Tensor, W_packed: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                     eps: float = 1e-5, gamma: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.float32, workspace: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None):
    """Z = LayerNorm(((X ⊙ b) W_sign^T) ⊙ a) through ``obl_linear_layernorm``.

    Returns (Z, workspace); the workspace holds the fp32 Y before normalisation."""
    M, K = _mat(X, "X")
    _dtype(X, "X", _XDT)
    N = _mat(W_packed, "W_packed")[0]
    _packed(W_packed, "W_packed", N, K)
    sdt = _scales([(a, "a", N), (b, "b", K)], None)
    gdt = _affine(gamma, beta, N)
    if gdt is not None and gdt != sdt:
        raise ValueError(f"gamma/beta have dtype {gdt}, the layer's scales {sdt}: they must match")
    workspace = _out(workspace, "workspace", (M, N), (torch.float32,), torch.float32, X.device)
    out = _out(out, "out", (M, N), _YDT, out_dtype, X.device)
    _check(lib.obl_linear_layernorm(_ptr(X), dtype_code(X.dtype), M, K, _ptr(W_packed), N, _ptr(a), _ptr(b),
                                    dtype_code(sdt), eps, _ptr(gamma), _ptr(beta), _ptr(workspace),
                                    _ptr(out), dtype_code(out.dtype), _stream(X)), "obl_linear_layernorm")
    return out, workspace


# ---------------------------------------------------------------------------
# Measurement hooks for the benchmark (internal exports, not part of obl.h).
def linear_span(X: torch.Tensor, W_packed: torch.Tensor, a: torch.Tensor, b: torch.Tensor, out: torch.Tensor,
                span: torch.Tensor) -> torch.Tensor:
    """``linear`` whose decode-GEMV launch (M <= 2) also records, per workgroup, its start and end in
    constant-clock ticks into ``span`` (int64, at least 2 N entries, 16-byte aligned)."""
    M, K = _mat(X, "X")
    _dtype(X, "X", _XDT)
    N = _mat(W_packed, "W_packed")[0]
    _packed(W_packed, "W_packed", N, K)
    sdt = _scales([(a, "a", N), (b, "b", K)], None)
    out = _out(out, "out", (M, N), _YDT, torch.float32, X.device)
    _dev(span, "span")
    _dtype(span, "span", (torch.int64,))
    if span.numel() < 2 * N:
        raise ValueError("span must hold 2 N entries")
    _check(lib.obl_internal_linear_span(_ptr(X), dtype_code(X.dtype), M, K, _ptr(W_packed), N, _ptr(a), _ptr(b),
                                        dtype_code(sdt), _ptr(out), dtype_code(out.dtype), _ptr(span), _stream(X)),
           "obl_internal_linear_span")
    return out


def peak_read(buf: torch.Tensor, sink: torch.Tensor):
    """Streaming read of every byte of ``buf`` (measurement kernel); ``sink`` (int32, >= 8 per CU) is
    never written in practice."""
    _dev(buf, "buf")
    _dev(sink, "sink")
    _check(lib.obl_internal_peak_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(buf)),
           "obl_internal_peak_read")


def peak_mfma(iters: int, sink: torch.Tensor) -> float:
    """Matrix-core loop (measurement kernel); returns the launch's dense flop count.  ``sink`` (fp32,
    >= 512 per CU) is never written in practice."""
    _dev(sink, "sink")
    flops = ctypes.c_double(0.0)
    _check(lib.obl_internal_peak_mfma(iters, _ptr(sink), ctypes.byref(flops), _stream(sink)), "obl_internal_peak_mfma")
    return flops.value
