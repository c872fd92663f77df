"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before touching HIP (so these run without a GPU).

Pointers here are fake addresses: every call below fails validation (or is the
M = 0 no-op) before any HIP call, so nothing is dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "obl.h")

b = pytest.importorskip("bit_weight_linear_amd.binding", reason="libobl.so not built")
L = b.lib
P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(obl_\w+|dbf_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("obl_pack_signs", "obl_linear", "dbf_linear"):
        assert n in names


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(L, name), f"{name} not exported"
    assert set(declared_functions()) == set(b.EXPORTS)


def test_status_strings_and_version():
    for code in range(11):
        assert L.obl_status_string(code) != b"OBL_ERR_UNKNOWN"
    assert L.obl_status_string(99) == b"OBL_ERR_UNKNOWN"
    assert L.obl_version() >= 100


# Fake but aligned, non-overlapping device addresses.
X, W, A, B_, Y, WS, S1 = (P(0x10_0000_0000 * (i + 1)) for i in range(7))


def lin(X=X, xd=b.OBL_BF16, M=1, K=4096, W=W, N=11008, a=A, bb=B_, sd=b.OBL_F16, Y=Y, yd=b.OBL_F32):
    return L.obl_linear(X, xd, M, K, W, N, a, bb, sd, Y, yd, None)


def test_linear_valid_m0_is_noop():
    assert lin(M=0) == b.OBL_OK
    assert lin(M=0, X=None, Y=None) == b.OBL_OK


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), b.OBL_ERR_NULL),
    (dict(a=None), b.OBL_ERR_NULL),
    (dict(bb=None), b.OBL_ERR_NULL),
    (dict(X=None), b.OBL_ERR_NULL),
    (dict(Y=None), b.OBL_ERR_NULL),
    (dict(M=-1), b.OBL_ERR_SHAPE),
    (dict(K=0), b.OBL_ERR_SHAPE),
    (dict(K=100), b.OBL_ERR_SHAPE),
    (dict(N=0), b.OBL_ERR_SHAPE),
    (dict(M=1 << 40, K=1 << 30), b.OBL_ERR_SHAPE),
    (dict(M=1 << 31, K=32, N=1), b.OBL_ERR_SHAPE),          # dimension beyond int32
    (dict(M=1, K=1 << 31, N=1), b.OBL_ERR_SHAPE),
    (dict(M=1, K=32, N=1 << 31), b.OBL_ERR_SHAPE),
    (dict(xd=b.OBL_I8), b.OBL_ERR_DTYPE),
    (dict(xd=b.OBL_F16), b.OBL_ERR_DTYPE),
    (dict(sd=b.OBL_BF16), b.OBL_ERR_DTYPE),
    (dict(yd=b.OBL_F16), b.OBL_ERR_DTYPE),
    (dict(yd=7), b.OBL_ERR_DTYPE),
    (dict(X=P(0x10_0000_0001)), b.OBL_ERR_ALIGN),
    (dict(W=P(0x20_0000_0002)), b.OBL_ERR_ALIGN),
    (dict(Y=P(0x50_0000_0002)), b.OBL_ERR_ALIGN),
    (dict(Y=P(0x10_0000_0000 + 4096)), b.OBL_ERR_ALIAS),      # Y inside X
    (dict(Y=P(0x20_0000_0000 + 1024)), b.OBL_ERR_ALIAS),      # Y inside W
    (dict(a=P(0x50_0000_0000 + 8)), b.OBL_ERR_ALIAS),         # a inside Y
])
def test_linear_rejects(kw, code):
    assert lin(**kw) == code


def test_forced_path_must_fit_m(forcer):
    forcer(path="lut")
    assert lin(M=3) == b.OBL_ERR_SHAPE
    forcer(path="decode")
    assert lin(M=33) == b.OBL_ERR_SHAPE
    # 17..32 rows only on the whole-K kernel (bf16 x, fp16 scales, aligned):
    # fp32 x, or a K that is not a multiple of 128, is refused before any GPU work
    assert lin(M=17, xd=b.OBL_F32) == b.OBL_ERR_SHAPE
    assert lin(M=17, K=96) == b.OBL_ERR_SHAPE
    assert lin(M=0) == b.OBL_OK


def dbf(X=X, M=8, K=4096, S2=W, Kmid=3072, S1_=S1, N=4096, bb=B_, m=A, a=P(0x80_0000_0000),
        sd=b.OBL_F16, ws=WS, Y=Y, yd=b.OBL_F32, xd=b.OBL_BF16):
    return L.dbf_linear(X, xd, M, K, S2, Kmid, S1_, N, bb, m, a, sd, ws, Y, yd, None)


def test_dbf_m0_noop():
    assert dbf(M=0) == b.OBL_OK


@pytest.mark.parametrize("kw,code", [
    (dict(S2=None), b.OBL_ERR_NULL),
    (dict(S1_=None), b.OBL_ERR_NULL),
    (dict(m=None), b.OBL_ERR_NULL),
    (dict(ws=None), b.OBL_ERR_NULL),
    (dict(Kmid=100), b.OBL_ERR_SHAPE),
    (dict(Kmid=0), b.OBL_ERR_SHAPE),
    (dict(K=48), b.OBL_ERR_SHAPE),
    (dict(sd=b.OBL_I8), b.OBL_ERR_DTYPE),
    (dict(ws=P(0x60_0000_0002)), b.OBL_ERR_ALIGN),
    (dict(ws=P(0x10_0000_0000 + 64)), b.OBL_ERR_ALIAS),        # workspace inside X
    (dict(ws=P(0x50_0000_0000)), b.OBL_ERR_ALIAS),             # workspace == Y
    (dict(Y=P(0x30_0000_0000 + 4)), b.OBL_ERR_ALIAS),          # Y inside a
])
def test_dbf_rejects(kw, code):
    assert dbf(**kw) == code


def dbf_noalloc(X=X, M=8, K=4096, S2=W, Kmid=3072, S1_=S1, N=4096, bb=B_, m=A, a=P(0x80_0000_0000),
                sd=b.OBL_F16, ws=WS, Y=Y, yd=b.OBL_F32, xd=b.OBL_BF16):
    return L.dbf_linear_noalloc(X, xd, M, K, S2, Kmid, S1_, N, bb, m, a, sd, ws, Y, yd, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), b.OBL_OK),
    (dict(S2=None), b.OBL_ERR_NULL),
    (dict(Kmid=100), b.OBL_ERR_SHAPE),
    (dict(sd=b.OBL_I8), b.OBL_ERR_DTYPE),
    (dict(ws=P(0x60_0000_0002)), b.OBL_ERR_ALIGN),
    (dict(ws=P(0x50_0000_0000)), b.OBL_ERR_ALIAS),
])
def test_dbf_noalloc_validates_like_dbf_linear(kw, code):
    assert dbf_noalloc(**kw) == code == dbf(**kw)


@pytest.mark.parametrize("args,code", [
    ((None, b.OBL_I8, 4, 64, W), b.OBL_ERR_NULL),
    ((X, b.OBL_I8, 4, 64, None), b.OBL_ERR_NULL),
    ((X, b.OBL_I8, 0, 64, W), b.OBL_ERR_SHAPE),
    ((X, b.OBL_I8, 4, 48, W), b.OBL_ERR_SHAPE),
    ((X, 9, 4, 64, W), b.OBL_ERR_DTYPE),
    ((P(0x10_0000_0002), b.OBL_F32, 4, 64, W), b.OBL_ERR_ALIGN),
    ((X, b.OBL_I8, 4, 64, P(0x10_0000_0000 + 32)), b.OBL_ERR_ALIAS),
])
def test_pack_rejects(args, code):
    assert L.obl_pack_signs(*args, None) == code


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        b.pack_signs(torch.ones((2, 32), dtype=torch.int8))


@pytest.mark.parametrize("args,code", [
    ((None, 64, 64, W), b.OBL_ERR_NULL),
    ((X, 64, 64, None), b.OBL_ERR_NULL),
    ((X, 48, 64, W), b.OBL_ERR_SHAPE),          # rows not a multiple of 32
    ((X, 64, 40, W), b.OBL_ERR_SHAPE),
    ((X, 0, 64, W), b.OBL_ERR_SHAPE),
    ((P(0x10_0000_0002), 64, 64, W), b.OBL_ERR_ALIGN),
    ((X, 64, 64, P(0x10_0000_0000 + 32)), b.OBL_ERR_ALIAS),
])
def test_transpose_rejects(args, code):
    assert L.obl_transpose_signs(*args, None) == code


# obl_linear_backward(dY, X, xd, M, K, W, Wt, N, a, b, sd, dX, dxd, da, db, ws, stream)
GY, WT, DX, DA, DB = (P(0x90_0000_0000 + 0x10_0000_0000 * i) for i in range(5))


def bwd(dY=GY, X_=X, xd=b.OBL_BF16, M=4, K=4096, W_=W, Wt=WT, N=4096, a=A, bb=B_, sd=b.OBL_F16,
        dX=DX, dxd=b.OBL_F32, da=DA, db=DB, ws=WS):
    return L.obl_linear_backward(dY, X_, xd, M, K, W_, Wt, N, a, bb, sd, dX, dxd, da, db, ws, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Wt=None), b.OBL_ERR_NULL),
    (dict(da=None), b.OBL_ERR_NULL),
    (dict(ws=None), b.OBL_ERR_NULL),
    (dict(N=4016), b.OBL_ERR_SHAPE),            # N must be a multiple of 32 (contraction of dX)
    (dict(K=4016), b.OBL_ERR_SHAPE),
    (dict(M=-1), b.OBL_ERR_SHAPE),
    (dict(xd=b.OBL_F16), b.OBL_ERR_DTYPE),
    (dict(dxd=b.OBL_I8), b.OBL_ERR_DTYPE),
    (dict(da=P(0xB0_0000_0002)), b.OBL_ERR_ALIGN),
    (dict(dX=P(0x10_0000_0000 + 64)), b.OBL_ERR_ALIAS),     # dX inside X
    (dict(db=DA), b.OBL_ERR_ALIAS),                          # two outputs overlap
    (dict(ws=GY), b.OBL_ERR_ALIAS),                          # workspace == dY
])
def test_backward_rejects(kw, code):
    assert bwd(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((None, b.OBL_F16, 64, 64, 8, W, A, B_), b.OBL_ERR_NULL),
    ((X, b.OBL_F16, 64, 64, 8, None, A, B_), b.OBL_ERR_NULL),
    ((X, b.OBL_F16, 64, 48, 8, W, A, B_), b.OBL_ERR_SHAPE),
    ((X, b.OBL_F16, 0, 64, 8, W, A, B_), b.OBL_ERR_SHAPE),
    ((X, b.OBL_F16, 64, 64, 0, W, A, B_), b.OBL_ERR_SHAPE),
    ((X, b.OBL_I8, 64, 64, 8, W, A, B_), b.OBL_ERR_DTYPE),
    ((P(0x10_0000_0001), b.OBL_F16, 64, 64, 8, W, A, B_), b.OBL_ERR_ALIGN),
    ((X, b.OBL_F16, 64, 64, 8, P(0x10_0000_0000 + 64), A, B_), b.OBL_ERR_ALIAS),
    ((X, b.OBL_F16, 64, 64, 8, W, A, A), b.OBL_ERR_ALIAS),
])
def test_svid_rejects(args, code):
    assert L.obl_svid(*args, b.OBL_F16, None) == code


# ------------------------------------------------------------------ LayerNorm
G_, BT = P(0x80_0000_0000), P(0x90_0000_0000)


def ln(Y=Y, yd=b.OBL_F32, M=4, N=4096, eps=1e-5, g=G_, be=BT, gd=b.OBL_F16, Z=WS, zd=b.OBL_BF16):
    return L.obl_layernorm(Y, yd, M, N, eps, g, be, gd, Z, zd, None)


def test_layernorm_m0_is_noop():
    assert ln(M=0) == b.OBL_OK
    assert ln(M=0, Y=None, Z=None) == b.OBL_OK


@pytest.mark.parametrize("kw,code", [
    (dict(Y=None), b.OBL_ERR_NULL),
    (dict(Z=None), b.OBL_ERR_NULL),
    (dict(M=-1), b.OBL_ERR_SHAPE),
    (dict(N=0), b.OBL_ERR_SHAPE),
    (dict(M=1 << 40, N=1 << 30), b.OBL_ERR_SHAPE),
    (dict(M=1 << 31, N=1), b.OBL_ERR_SHAPE),
    (dict(M=1, N=1 << 31), b.OBL_ERR_SHAPE),
    (dict(yd=b.OBL_F16), b.OBL_ERR_DTYPE),
    (dict(zd=b.OBL_I8), b.OBL_ERR_DTYPE),
    (dict(gd=b.OBL_BF16), b.OBL_ERR_DTYPE),
    (dict(eps=-1.0), b.OBL_ERR_VALUE),
    (dict(eps=float("nan")), b.OBL_ERR_VALUE),
    (dict(eps=float("inf")), b.OBL_ERR_VALUE),
    (dict(Y=P(0x50_0000_0002)), b.OBL_ERR_ALIGN),
    (dict(Z=P(0x60_0000_0001)), b.OBL_ERR_ALIGN),
    (dict(g=P(0x80_0000_0001)), b.OBL_ERR_ALIGN),
    (dict(Z=P(0x50_0000_0000 + 64)), b.OBL_ERR_ALIAS),     # Z inside Y
    (dict(g=P(0x60_0000_0000 + 64)), b.OBL_ERR_ALIAS),     # gamma inside Z
    (dict(be=P(0x60_0000_0000 + 64)), b.OBL_ERR_ALIAS),    # beta inside Z
])
def test_layernorm_rejects(kw, code):
    assert ln(**kw) == code


def test_layernorm_affine_dtype_ignored_without_affine():
    # No gamma/beta: the affine dtype is not checked; M = 0 keeps it a no-op.
    assert ln(M=0, g=None, be=None, gd=b.OBL_BF16) == b.OBL_OK


def lln(X=X, xd=b.OBL_BF16, M=2, K=4096, W=W, N=4096, a=A, bb=B_, sd=b.OBL_F16, eps=1e-5, g=G_, be=BT,
        ws=S1, Z=WS, zd=b.OBL_F32):
    return L.obl_linear_layernorm(X, xd, M, K, W, N, a, bb, sd, eps, g, be, ws, Z, zd, None)


def test_linear_layernorm_m0_is_noop():
    assert lln(M=0) == b.OBL_OK
    assert lln(M=0, X=None, ws=None, Z=None) == b.OBL_OK


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), b.OBL_ERR_NULL),
    (dict(ws=None), b.OBL_ERR_NULL),
    (dict(Z=None), b.OBL_ERR_NULL),
    (dict(K=100), b.OBL_ERR_SHAPE),
    (dict(xd=b.OBL_F16), b.OBL_ERR_DTYPE),
    (dict(sd=b.OBL_BF16), b.OBL_ERR_DTYPE),
    (dict(zd=b.OBL_F16), b.OBL_ERR_DTYPE),
    (dict(eps=-0.5), b.OBL_ERR_VALUE),
    (dict(ws=P(0x70_0000_0002)), b.OBL_ERR_ALIGN),
    (dict(ws=P(0x10_0000_0000 + 256)), b.OBL_ERR_ALIAS),    # workspace inside X
    (dict(ws=P(0x80_0000_0000 - 64)), b.OBL_ERR_ALIAS),     # workspace over gamma
    (dict(Z=P(0x70_0000_0000 + 64)), b.OBL_ERR_ALIAS),      # Z inside workspace
    (dict(Z=P(0x20_0000_0000 + 64)), b.OBL_ERR_ALIAS),      # Z inside W
])
def test_linear_layernorm_rejects(kw, code):
    assert lln(**kw) == code


def test_every_call_rejects_dimensions_beyond_int32():
    big = 1 << 31
    assert L.obl_pack_signs(X, b.OBL_I8, big, 32, W, None) == b.OBL_ERR_SHAPE
    assert L.obl_transpose_signs(W, big, 32, Y, None) == b.OBL_ERR_SHAPE
    assert L.obl_svid(X, b.OBL_F16, big, 32, 4, W, A, B_, b.OBL_F16, None) == b.OBL_ERR_SHAPE
    assert L.dbf_linear(X, b.OBL_BF16, 1, 32, W, big, S1, 32, A, B_, Y, b.OBL_F16, WS, P(0x80_0000_0000),
                        b.OBL_F32, None) == b.OBL_ERR_SHAPE
    assert L.obl_linear_backward(X, Y, b.OBL_BF16, 1, 32, W, S1, big, A, B_, b.OBL_F16, WS, b.OBL_F32,
                                 P(0x80_0000_0000), P(0x90_0000_0000), P(0xA0_0000_0000), None) == b.OBL_ERR_SHAPE
    assert L.obl_linear_layernorm(X, b.OBL_BF16, big, 32, W, 32, A, B_, b.OBL_F16, 1e-5, None, None, WS, Y,
                                  b.OBL_F32, None) == b.OBL_ERR_SHAPE
