"""Plain, slow, obviously-correct fp64 oracle.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this module.  The HIP library never does, and this module never
imports the library.

Sources (the reader has the pages, cited by title and section):

* OneBit page -- "1bit量化" (blog.zerodtree.com), a walk-through of the OneBit
  paper: "rank-1 approximation", the sign/value split, "proposition 1" and its
  proof, "lemma 1", "proposition 2", and the "知识蒸馏" block that restates the
  layer with ``g`` and ``h``.
* DBF page -- "Addition is almost all you need: Compressing large language
  models with double binary factorization" (gist.science summary),
  "Technische samenvatting / Methodologie: Double Binary Factorization".

Conventions (OneBit page, proposition 1 proof, which writes X W^T with W
indexed [output, input]): ``X`` is [M, K], a weight or sign matrix is [N, K],
``a`` has N entries (output side, the architecture's ``h``) and ``b`` has K
entries (input side, the architecture's ``g``).  DBF: ``S1`` (the page's
A with entries +-1) is [N, Kmid], ``S2`` (the page's B) is [Kmid, K], ``m`` has
Kmid entries.

Packed sign format (the pages fix none; this is the reading every part of the
project uses): ``P[r, w]`` is a uint32 whose bit ``j`` (LSB = bit 0) holds the
sign of column ``32*w + j`` of row ``r``; bit value 1 means -1, 0 means +1.
``Sign`` of zero (the pages give no tie-break, and zero does not fit one bit)
packs as +1: only values strictly below zero pack as -1.

Parity status: every public function here is pinned by ``tests/test_oracle.py``
(page values, closed forms, brute force, library special cases); none is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "sign_pm1",
    "pack_signs",
    "unpack_signs",
    "onebit_dense_weight",
    "onebit_linear",
    "onebit_error_scale",
    "dbf_dense_weight",
    "dbf_linear",
    "dbf_stage1",
    "dbf_error_scale",
    "power_iteration_sigma1",
    "rank1_power",
    "svid",
    "max_normalised_error",
    "transpose_signs",
    "onebit_backward",
    "backward_error_scales",
    "layernorm_rows",
]


def _f64(x) -> np.ndarray:
    """Upcast to float64 (exact for fp16, bf16 and fp32 values)."""
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Sign matrices and the packed format
# --------------------------------------------------------------------------
def sign_pm1(W) -> np.ndarray:
    """``W_sign = Sign(W)`` (OneBit page, the split W = W_sign ⊙ |W|), as int8 +-1.

    Zero (and -0.0, NaN) maps to +1: only ``w < 0`` gives -1.
    """
    W = np.asarray(W)
    return np.where(W < 0, -1, 1).astype(np.int8)


def pack_signs(S) -> np.ndarray:
    """Pack a +-1 (or any real) matrix [R, K] into uint32 words [R, K/32].

    Bit j of word w is 1 exactly when ``S[r, 32*w + j] < 0``.  Written as a
    plain loop over the 32 bit positions.
    """
    S = np.asarray(S)
    if S.ndim != 2:
        raise ValueError("pack_signs expects a 2-D matrix")
    R, K = S.shape
    if K % 32 != 0:
        raise ValueError("K must be a multiple of 32")
    neg = (S < 0).reshape(R, K // 32, 32)
    out = np.zeros((R, K // 32), dtype=np.uint64)
    for j in range(32):
        out |= neg[:, :, j].astype(np.uint64) << np.uint64(j)
    return out.astype(np.uint32)


def unpack_signs(P, K: int) -> np.ndarray:
    """Inverse of :func:`pack_signs`: uint32 [R, K/32] -> int8 +-1 [R, K]."""
    P = np.asarray(P, dtype=np.uint32)
    R, W = P.shape
    if W * 32 != K:
        raise ValueError("packed width does not match K")
    S = np.empty((R, K), dtype=np.int8)
    for j in range(32):
        bit = (P >> np.uint32(j)) & np.uint32(1)
        S[:, j::32] = np.where(bit == 1, -1, 1)
    return S


# --------------------------------------------------------------------------
# OneBit layer
# --------------------------------------------------------------------------
def onebit_dense_weight(W_sign, a, b) -> np.ndarray:
    """Dense weight of the sign/value split: ``W = W_sign ⊙ (a b^T)``.

    OneBit page, "rank-1 approximation" block (W ≈ W_sign ⊙ (a b^T)) and the
    first line of the proposition 1 proof (w_jk = s_jk · a_j · b_k).
    Exact in fp64 for fp16/bf16/fp32 scales.
    """
    S = _f64(W_sign)
    a = _f64(a)
    b = _f64(b)
    N, K = S.shape
    if a.shape != (N,) or b.shape != (K,):
        raise ValueError("a must have N entries and b must have K entries")
    return S * a[:, None] * b[None, :]


def onebit_linear(X, W_sign, a, b) -> np.ndarray:
    """``Y = X W^T`` with the dense ``W`` above (OneBit page, proposition 1).

    Proposition 1 states that this product equals
    ``[(X ⊙ b^T) W_sign^T] ⊙ a^T``; given (W_sign, a, b) the two sides are the
    same number (associativity), so the oracle evaluates the plain definition:
    form W densely, then one fp64 matrix product.
    """
    X = _f64(X)
    W = onebit_dense_weight(W_sign, a, b)
    if X.ndim != 2 or X.shape[1] != W.shape[1]:
        raise ValueError("X must be [M, K]")
    return X @ W.T


def onebit_error_scale(X, a, b) -> np.ndarray:
    """Normalising scale ``S[i, j] = |a_j| · Σ_k |x_ik b_k|`` (fp64).

    The tolerance of a computed ``Y`` is expressed as a multiple of this
    quantity: it bounds ``|Y_ij|`` and every partial sum of the contraction.
    """
    X = _f64(X)
    a = _f64(a)
    b = _f64(b)
    return np.abs(X) @ np.abs(b)[:, None] * np.abs(a)[None, :]


# --------------------------------------------------------------------------
# Double Binary Factorization
# --------------------------------------------------------------------------
def dbf_dense_weight(S1, S2, a, m, b) -> np.ndarray:
    """``W = (a ⊙ A ⊙ m^T)(B ⊙ b^T)`` with A = S1 [N, Kmid], B = S2 [Kmid, K].

    DBF page, "Methodologie": the factorisation of W into two +-1 matrices with
    the scale vectors a, m, b.
    """
    S1 = _f64(S1)
    S2 = _f64(S2)
    a = _f64(a)
    m = _f64(m)
    b = _f64(b)
    N, Kmid = S1.shape
    Kmid2, K = S2.shape
    if Kmid2 != Kmid or a.shape != (N,) or m.shape != (Kmid,) or b.shape != (K,):
        raise ValueError("inconsistent DBF shapes")
    left = a[:, None] * S1 * m[None, :]
    right = S2 * b[None, :]
    return left @ right


def dbf_linear(X, S1, S2, a, m, b) -> np.ndarray:
    """``Y = X W^T`` for the DBF weight above (DBF page, "Methodologie").

    The page's inference chain ``((((X ⊙ b^T) B^T) ⊙ m^T) A^T) ⊙ a^T`` is the
    same number given the factors; the oracle evaluates the plain definition.
    """
    X = _f64(X)
    return X @ dbf_dense_weight(S1, S2, a, m, b).T


def dbf_stage1(X, S2, b, m) -> np.ndarray:
    """Inner part of the DBF chain, ``T1 = ((X ⊙ b^T) B^T) ⊙ m^T`` [M, Kmid].

    It is a OneBit layer with sign matrix B, input scale b and output scale m,
    so the OneBit definition is reused.
    """
    return onebit_linear(X, S2, m, b)


def dbf_error_scale(X, b, m, a) -> np.ndarray:
    """``S_dbf[i, j] = |a_j| · (Σ_l |m_l|) · Σ_k |x_ik b_k|``: bounds |Y| and
    every partial sum through both stages (triangle inequality)."""
    X = _f64(X)
    base = np.abs(X) @ np.abs(_f64(b))
    return base[:, None] * np.abs(_f64(m)).sum() * np.abs(_f64(a))[None, :]


# --------------------------------------------------------------------------
# Backward of the OneBit layer (OneBit page, "知识蒸馏": the layer
# Y = [(X ⊙ g) W_±1^T] ⊙ h is trained by distillation, so its input and scale
# gradients are needed; they follow from the plain definition by the chain rule.)
# --------------------------------------------------------------------------
def transpose_signs(P, rows: int, K: int) -> np.ndarray:
    """Packed signs of the transposed sign matrix: ``P^T`` [K, rows/32] from
    ``P`` [rows, K/32] (same packing format, now along the ``rows`` axis)."""
    return pack_signs(unpack_signs(P, K).T)


def onebit_backward(X, W_sign, a, b, dY):
    """Gradients of ``Y = X W^T`` with ``W = W_sign ⊙ (a b^T)`` for an upstream
    gradient ``dY`` [M, N]: returns ``(dX, da, db)``.

    ``dX = dY W``; with ``dW = dY^T X`` the scale gradients are
    ``da_j = Σ_k dW_jk s_jk b_k`` and ``db_k = Σ_j dW_jk s_jk a_j`` (the signs
    themselves are fixed and get no gradient).
    """
    X = _f64(X)
    dY = _f64(dY)
    S = _f64(W_sign)
    a = _f64(a)
    b = _f64(b)
    W = onebit_dense_weight(S, a, b)
    dX = dY @ W
    dW = dY.T @ X
    da = (dW * S * b[None, :]).sum(axis=1)
    db = (dW * S * a[:, None]).sum(axis=0)
    return dX, da, db


def backward_error_scales(X, a, b, dY):
    """Normalising scales bounding every partial sum of each gradient:
    ``S_dX[i, k] = |b_k| Σ_j |dY_ij a_j|``, ``S_da[j] = Σ_i |dY_ij| Σ_k |x_ik b_k|``,
    ``S_db[k] = Σ_i |x_ik| Σ_j |dY_ij a_j|``."""
    X = _f64(X)
    dY = _f64(dY)
    a = np.abs(_f64(a))
    b = np.abs(_f64(b))
    ga = np.abs(dY) @ a                    # [M]: Σ_j |dY_ij a_j|
    xb = np.abs(X) @ b                     # [M]: Σ_k |x_ik b_k|
    s_dx = ga[:, None] * b[None, :]
    s_da = np.abs(dY).T @ xb
    s_db = np.abs(X).T @ ga
    return s_dx, s_da, s_db


# --------------------------------------------------------------------------
# LayerNorm after the layer (OneBit page, "知识蒸馏" block: Z = LayerNorm(Y)).
# The page gives neither epsilon nor affine parameters; the reading used is the
# textbook per-row normalisation with a caller-given epsilon (1e-5 by default)
# and optional elementwise gamma, beta.
# --------------------------------------------------------------------------
def layernorm_rows(Y, eps: float = 1e-5, gamma=None, beta=None) -> np.ndarray:
    """``z_ij = (y_ij - mean_i) / sqrt(var_i + eps) * gamma_j + beta_j`` with the
    row mean and the biased (population) row variance."""
    Y = _f64(Y)
    mu = Y.mean(axis=1, keepdims=True)
    var = ((Y - mu) ** 2).mean(axis=1, keepdims=True)
    Z = (Y - mu) / np.sqrt(var + eps)
    if gamma is not None:
        Z = Z * _f64(gamma)[None, :]
    if beta is not None:
        Z = Z + _f64(beta)[None, :]
    return Z


# --------------------------------------------------------------------------
# Rank-1 machinery (OneBit page: rank-1 approximation, lemma 1, proposition 2)
# --------------------------------------------------------------------------
def rank1_power(A, iters: int = 20000, tol: float = 1e-15, seed: int = 1234):
    """Leading singular triple ``(σ1, u1, v1)`` of A by power iteration on A^T A.

    OneBit page, "rank-1 approximation": the best rank-1 approximation in
    Frobenius norm keeps the largest singular value and its two singular
    vectors (û = u1 σ1 v1^T).  The start vector is seeded so results repeat.
    """
    A = _f64(A)
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(A.shape[1])
    v /= np.linalg.norm(v)
    sigma = 0.0
    for _ in range(iters):
        w = A.T @ (A @ v)
        nw = np.linalg.norm(w)
        if nw == 0.0:
            return 0.0, np.zeros(A.shape[0]), v
        v_new = w / nw
        sigma_new = float(np.linalg.norm(A @ v_new))
        done = abs(sigma_new - sigma) <= tol * max(sigma_new, 1e-300)
        v, sigma = v_new, sigma_new
        if done:
            break
    u = A @ v
    nu = np.linalg.norm(u)
    u = u / nu if nu > 0 else u
    return sigma, u, v


def power_iteration_sigma1(A, **kw) -> float:
    """σ1(A) (the induced 2-norm, OneBit page lemma 1 proof) by power iteration."""
    return rank1_power(A, **kw)[0]


def svid(W):
    """Sign-Value-Independent Decomposition: ``W ≈ W_sign ⊙ (a b^T)``.

    OneBit page, "rank-1 approximation" block: W_sign = Sign(W), and the rank-1
    approximation of |W| gives a b^T.  The split of σ1 between a and b is not
    given; the reading used is a = sqrt(σ1)·u1, b = sqrt(σ1)·v1 with the
    singular vectors taken nonnegative (|W| is entrywise nonnegative, so its
    leading singular vectors can be).
    """
    W = _f64(W)
    sigma, u, v = rank1_power(np.abs(W))
    if u.sum() < 0:
        u = -u
    if v.sum() < 0:
        v = -v
    root = np.sqrt(sigma)
    return sign_pm1(W), root * np.abs(u), root * np.abs(v)


# --------------------------------------------------------------------------
# Verdict helper
# --------------------------------------------------------------------------
def max_normalised_error(Y, Y_ref, S) -> float:
    """``max_ij |Y_ij - Y_ref_ij| / S_ij`` (0/0 counts as 0)."""
    Y = _f64(Y)
    Y_ref = _f64(Y_ref)
    S = _f64(S)
    diff = np.abs(Y - Y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(S > 0, diff / np.where(S > 0, S, 1.0), np.where(diff > 0, np.inf, 0.0))
    return float(r.max()) if r.size else 0.0
