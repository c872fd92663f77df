"""Degenerate inputs of the sign-binarised layer, checked against closed forms
that need neither the oracle nor the dense weight matrix.

OneBit page, proposition 1: Y = [(X ⊙ bᵀ) W_signᵀ] ⊙ aᵀ.  Special cases:
  * every sign +1 (packed words all zero):  Y_mn = a_n Σ_k x_mk b_k;
  * every sign -1 (packed words all ones):  Y_mn = -a_n Σ_k x_mk b_k;
  * X = 0, or a = 0, or b = 0:               Y = 0 exactly;
  * one nonzero input x_mk (one-hot rows):   Y_mn = s_nk x_mk b_k a_n, one product,
    so every path returns the correctly rounded value when b is representable
    in bf16 (the matrix-core path rounds b to bf16; integer-valued b is exact).
Every path is run: the LUT GEMV (M <= 2), the decode kernels (M <= 16, split
and whole-K) and the prefill GEMM (M > 16), and the DBF layer with both
factors all +1."""
import numpy as np
import pytest
import torch

from bit_weight_linear_amd import workloads as WL
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

B = pytest.importorskip("bit_weight_linear_amd.binding", reason="libobl.so not built")

# (path, M, decode kernel or None): LUT at 1 and 2 rows, decode split and
# whole-K at 8 and 16 rows, prefill at 64 and 300 rows.
PATHS = [("lut", 1, None), ("lut", 2, None), ("decode", 8, "split"), ("decode", 16, "wk1"),
         ("decode", 5, "auto"), ("gemm", 64, None), ("gemm", 300, None)]
TOL = {"lut": G.TOL_DECODE, "decode": G.TOL_DECODE, "gemm": G.TOL_GEMM}


def _inputs(M, K, N, rng, b_int=False):
    X = WL.round_to(rng.standard_normal((M, K)), "bf16")
    a = WL.round_to(np.abs(rng.standard_normal(N)) * 0.5 + 0.01, "f16")
    if b_int:
        b = rng.integers(1, 9, K).astype(np.float64)
    else:
        b = WL.round_to(np.abs(rng.standard_normal(K)) * 0.02 + 1e-3, "f16")
    return X, a, b


def _run(path, decode, X, Wp, a, b, y=torch.float32):
    with B.forced_kernels(path=path, decode=decode if decode else None):
        Y = B.linear(G.dev(X, "bf16"), Wp, G.dev(a, "f16"), G.dev(b, "f16"), out_dtype=y)
    torch.cuda.synchronize()
    return G.host64(Y)


@pytest.mark.parametrize("path,M,decode", PATHS)
@pytest.mark.parametrize("sign", [1, -1])
def test_constant_signs_closed_form(path, M, decode, sign):
    K, N = 1024, 300
    rng = np.random.default_rng(M + (sign > 0))
    X, a, b = _inputs(M, K, N, rng)
    # packed words: bit set = -1, so all zeros (+1) or all ones (-1, int32 -1)
    Wp = torch.full((N, K // 32), 0 if sign > 0 else -1, dtype=torch.int32, device="cuda")
    G.say(f"constant signs {sign:+d} {path} M={M}")
    Y = _run(path, decode, X, Wp, a, b)
    xb = X @ b                                          # Σ_k x_mk b_k, fp64
    ref = sign * np.outer(xb, a)
    scale = np.outer(np.abs(X) @ np.abs(b), np.abs(a))  # the normalised error scale
    err = np.abs(Y - ref) / scale
    assert err.max() <= TOL[path], f"max normalised error {err.max():.3e}"
    # every column of Y / a is the same row sum: columns agree to the same bound
    assert np.abs(Y / a[None, :] - sign * xb[:, None]).max() <= TOL[path] * (np.abs(X) @ np.abs(b)).max()


@pytest.mark.parametrize("path,M,decode", PATHS)
@pytest.mark.parametrize("zero", ["x", "a", "b"])
def test_zero_operand_gives_exact_zero(path, M, decode, zero):
    K, N = 512, 200
    rng = np.random.default_rng(7 * M)
    X, a, b = _inputs(M, K, N, rng)
    if zero == "x":
        X = np.zeros_like(X)
    elif zero == "a":
        a = np.zeros_like(a)
    else:
        b = np.zeros_like(b)
    S = np.where(rng.random((N, K)) < 0.5, 1, -1).astype(np.int8)
    Wp = B.pack_signs(G.signs_dev(S))
    G.say(f"zero {zero} {path} M={M}")
    for y in (torch.float32, torch.bfloat16):
        Y = _run(path, decode, X, Wp, a, b, y)
        assert np.array_equal(Y, np.zeros((M, N))), f"{zero} = 0 must give Y = 0 exactly"


@pytest.mark.parametrize("path,M,decode", PATHS)
def test_one_hot_rows_are_exact(path, M, decode):
    """One nonzero x per row: the contraction has a single term, so Y is the
    correctly rounded fp32 value of s·x·b·a (integer b: exact in bf16 too)."""
    K, N = 640, 257
    rng = np.random.default_rng(11 * M)
    _, a, b = _inputs(M, K, N, rng, b_int=True)
    X = np.zeros((M, K))
    cols = rng.integers(0, K, M)
    X[np.arange(M), cols] = WL.round_to(rng.standard_normal(M) * 4, "bf16")
    S = np.where(rng.random((N, K)) < 0.5, 1, -1).astype(np.int8)
    Wp = B.pack_signs(G.signs_dev(S))
    G.say(f"one-hot {path} M={M}")
    Y = _run(path, decode, X, Wp, a, b)
    # x·b is exact in fp32 (bf16 x, integer b <= 8); times a: one rounding
    xb = (X[np.arange(M), cols] * b[cols]).astype(np.float32)
    ref = (S[:, cols].T.astype(np.float32) * xb[:, None]) * a.astype(np.float32)[None, :]
    assert np.array_equal(Y, ref.astype(np.float64)), \
        f"max |diff| {np.abs(Y - ref).max():.3e} (one term per output must be exact)"


@pytest.mark.parametrize("M", [4, 8, 512])
def test_dbf_all_plus_signs_closed_form(M):
    """S2, S1 all +1: Y_mn = a_n (Σ_l m_l) (Σ_k x_mk b_k)."""
    K, Kmid, N = 1024, 768, 512
    rng = np.random.default_rng(M)
    X = WL.round_to(rng.standard_normal((M, K)), "bf16")
    b = WL.round_to(np.abs(rng.standard_normal(K)) + 0.1, "f16")
    m = WL.round_to(np.abs(rng.standard_normal(Kmid)) + 0.1, "f16")
    a = WL.round_to(np.abs(rng.standard_normal(N)) + 0.1, "f16")
    S2p = torch.zeros((Kmid, K // 32), dtype=torch.int32, device="cuda")
    S1p = torch.zeros((N, Kmid // 32), dtype=torch.int32, device="cuda")
    Y, _ = B.dbf_linear(G.dev(X, "bf16"), S2p, S1p, G.dev(b, "f16"), G.dev(m, "f16"), G.dev(a, "f16"))
    torch.cuda.synchronize()
    Y = G.host64(Y)
    ref = np.outer((X @ b) * m.sum(), a)
    scale = np.outer((np.abs(X) @ np.abs(b)) * np.abs(m).sum(), np.abs(a))
    tol = G.TOL_DECODE if M <= 16 else G.TOL_DBF_GEMM
    err = np.abs(Y - ref) / scale
    G.say(f"dbf all +1 M={M}: max normalised error {err.max():.3e}")
    assert err.max() <= tol
