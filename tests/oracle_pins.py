"""Pins that tie the fp64 oracle to something other than itself.

Each pin takes the oracle function(s) under test as arguments, so the same pin
runs against the real oracle (it must pass) and against planted mistakes
(``test_oracle.py`` checks that every planted mistake fails at least one pin).

What each pin compares against:
* page values  -- the LLM.int8() page's worked +-1 product (tests/golden/);
* closed forms -- Sylvester Hadamard H H^T = K I; DBF with S1 = S2 = H;
* a textbook routine -- the fast Walsh-Hadamard transform;
* exact integer arithmetic -- int64 matrix products in the integer-exact regime;
* brute force  -- pure-Python loops on tiny shapes;
* the pages' identities -- proposition 1 (dense vs factored form), the DBF
  factorisation vs its inference chain.
"""
from __future__ import annotations

import json
import os

import numpy as np

from bit_weight_linear_amd.workloads import random_signs, round_to, sylvester_hadamard

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _softmax_rows(Y):
    Y = np.asarray(Y, dtype=np.float64)
    e = np.exp(Y - Y.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def fwht_rows(X):
    """Fast Walsh-Hadamard transform of every row (natural / Sylvester order)."""
    Y = np.array(X, dtype=np.float64, copy=True)
    n = Y.shape[1]
    h = 1
    while h < n:
        for start in range(0, n, 2 * h):
            u = Y[:, start:start + h].copy()
            v = Y[:, start + h:start + 2 * h].copy()
            Y[:, start:start + h] = u + v
            Y[:, start + h:start + 2 * h] = u - v
        h *= 2
    return Y


# ---------------------------------------------------------------- packing
def pin_pack_patterns(pack, unpack):
    """Fixed bit patterns: all +1 -> 0, all -1 -> 0xFFFFFFFF, -1 at odd k -> 0xAAAAAAAA,
    a single -1 at column 32*w + j sets only bit j of word w."""
    errs = []
    S = np.ones((2, 64), dtype=np.int8)
    if not (pack(S) == 0).all():
        errs.append("all +1 must pack to 0")
    if not (pack(-S) == 0xFFFFFFFF).all():
        errs.append("all -1 must pack to 0xFFFFFFFF")
    alt = np.ones((1, 64), dtype=np.int8)
    alt[0, 1::2] = -1
    if not (pack(alt) == 0xAAAAAAAA).all():
        errs.append("-1 at odd k must pack to 0xAAAAAAAA")
    one = np.ones((1, 64), dtype=np.int8)
    one[0, 32 + 5] = -1
    p = pack(one)
    if not (p[0, 0] == 0 and p[0, 1] == (1 << 5)):
        errs.append("single -1 at column 37 must set bit 5 of word 1")
    for P, K in ((np.array([[0xAAAAAAAA]], dtype=np.uint32), 32),
                 (np.array([[1 << 5, 0x80000000]], dtype=np.uint32), 64)):
        ref = np.ones((1, K), dtype=np.int8)
        for w in range(K // 32):
            for j in range(32):
                if (int(P[0, w]) >> j) & 1:
                    ref[0, 32 * w + j] = -1
        if not (unpack(P, K) == ref).all():
            errs.append(f"unpack of {P.tolist()} wrong")
    rng = np.random.default_rng(7)
    S = random_signs(rng, (5, 96))
    if not (unpack(pack(S), 96) == S).all():
        errs.append("round trip failed")
    return errs


# ---------------------------------------------------------------- OneBit
def pin_page_pm1_example(onebit_linear):
    """LLM.int8() page, section 4.2.1: softmax(hidden @ pm1) = [0, .5, .5, 0] per row."""
    g = json.load(open(os.path.join(GOLDEN, "llm_int8_emergent_pm1_example.json")))
    H = np.array(g["hidden"], dtype=np.float64)
    P = np.array(g["pm1_matrix"], dtype=np.int8)
    Y = onebit_linear(H, P.T, np.ones(4), np.ones(4))      # X = hidden, W_sign = pm1^T
    got = np.round(_softmax_rows(Y), g["printed_decimals"])
    want = np.array(g["softmax_of_product"], dtype=np.float64)
    return [] if np.array_equal(got, want) else [f"page example: softmax {got.tolist()}"]


def pin_hadamard(onebit_linear):
    """Closed form H H^T = K I, and X H^T equals the fast Walsh-Hadamard transform."""
    errs = []
    for K in (32, 64, 512):
        H = sylvester_hadamard(K)
        Y = onebit_linear(H.astype(np.float64), H, np.ones(K), np.ones(K))
        if not np.array_equal(Y, K * np.eye(K)):
            errs.append(f"H H^T != {K} I")
        rng = np.random.default_rng(K)
        X = rng.standard_normal((3, K))
        if not np.allclose(onebit_linear(X, H, np.ones(K), np.ones(K)), fwht_rows(X),
                           rtol=0, atol=1e-12 * K):
            errs.append(f"X H^T != FWHT(X) at K={K}")
    return errs


def pin_scales_hadamard(onebit_linear):
    """With X = I and W_sign = H (non-symmetric shapes via a column slice):
    Y[i, j] = H[j, i] a_j b_i, so Y / (H^T) = outer(b, a) exactly (powers of two)."""
    K, N = 32, 16
    H = sylvester_hadamard(K)[:N]                  # [N, K]
    rng = np.random.default_rng(3)
    a = 2.0 ** rng.integers(-3, 4, size=N)
    b = 2.0 ** rng.integers(-3, 4, size=K)
    Y = onebit_linear(np.eye(K), H, a, b)          # [K, N]
    if Y.shape != (K, N):
        return [f"shape {Y.shape}"]
    ratio = Y / H.T.astype(np.float64)
    return [] if np.array_equal(ratio, np.outer(b, a)) else ["a/b placement wrong"]


def pin_int_exact(onebit_linear, seed=11):
    """Integer-exact regime: fp64 oracle equals an int64 matrix product exactly."""
    rng = np.random.default_rng(seed)
    errs = []
    for (M, K, N) in ((3, 64, 40), (5, 128, 33)):
        X = rng.integers(-2, 3, size=(M, K))
        S = random_signs(rng, (N, K)).astype(np.int64)
        ea = rng.integers(-1, 3, size=N)           # a = 2^ea
        eb = rng.integers(-1, 3, size=K)           # b = 2^eb
        # scale by 4 so every quantity is an integer: (X * 2b) @ S^T * 2a / 4
        xb = X * (2 ** (eb + 1))[None, :]
        T = xb @ S.T
        Y_int = T * (2 ** (ea + 1))[None, :]
        Y = onebit_linear(X.astype(np.float64), S.astype(np.int8), 2.0 ** ea, 2.0 ** eb)
        if not np.array_equal(Y * 4, Y_int.astype(np.float64)):
            errs.append(f"int-exact mismatch at {(M, K, N)}")
    return errs


def pin_bruteforce(onebit_linear, seed=5):
    """Pure-Python loops at M=4, N=8 (and K=8): y_ij = sum_k x_ik s_jk a_j b_k."""
    rng = np.random.default_rng(seed)
    M, K, N = 4, 8, 8
    X = rng.standard_normal((M, K))
    S = random_signs(rng, (N, K))
    a = rng.standard_normal(N)
    b = rng.standard_normal(K)
    Y = onebit_linear(X, S, a, b)
    errs = []
    for i in range(M):
        for j in range(N):
            acc = 0.0
            scale = 0.0
            for k in range(K):
                acc += float(X[i, k]) * int(S[j, k]) * float(a[j]) * float(b[k])
                scale += abs(float(X[i, k]) * float(a[j]) * float(b[k]))
            if abs(Y[i, j] - acc) > 1e-14 * scale:
                errs.append(f"brute force ({i},{j}) {Y[i, j]} vs {acc}")
    return errs


def pin_prop1_identity(onebit_linear, seed=9):
    """OneBit page, proposition 1: X W^T (dense W = W_sign ⊙ a b^T) equals
    [(X ⊙ b^T) W_sign^T] ⊙ a^T (evaluated here in that order), within 1e-12·S."""
    rng = np.random.default_rng(seed)
    errs = []
    for (M, K, N) in ((4, 64, 48), (7, 96, 96)):
        X = round_to(rng.standard_normal((M, K)), "bf16")
        S = random_signs(rng, (N, K))
        a = round_to(np.abs(rng.normal(0, 0.02, N)) + 1e-3, "f16")
        b = round_to(np.abs(rng.normal(0, 0.02, K)) + 1e-3, "f16")
        Y = onebit_linear(X, S, a, b)
        Yf = ((X * b[None, :]) @ S.T.astype(np.float64)) * a[None, :]
        scale = (np.abs(X) @ np.abs(b))[:, None] * np.abs(a)[None, :]
        if Y.shape != Yf.shape or (np.abs(Y - Yf) > 1e-12 * scale).any():
            errs.append(f"proposition 1 identity fails at {(M, K, N)}")
    return errs


ONEBIT_PINS = (pin_page_pm1_example, pin_hadamard, pin_scales_hadamard, pin_int_exact,
               pin_bruteforce, pin_prop1_identity)


# ---------------------------------------------------------------- DBF
def pin_dbf_chain(dbf_linear, seed=21):
    """DBF page: the factorisation (a ⊙ A ⊙ m^T)(B ⊙ b^T) and the inference chain
    ((((X ⊙ b^T) B^T) ⊙ m^T) A^T) ⊙ a^T agree within 1e-12·S_dbf."""
    rng = np.random.default_rng(seed)
    errs = []
    for (M, K, Kmid, N) in ((3, 64, 32, 40), (8, 96, 64, 64)):
        X = rng.standard_normal((M, K))
        S2 = random_signs(rng, (Kmid, K)).astype(np.float64)
        S1 = random_signs(rng, (N, Kmid)).astype(np.float64)
        b, m, a = (np.abs(rng.standard_normal(n)) + 0.1 for n in (K, Kmid, N))
        Y = dbf_linear(X, S1, S2, a, m, b)
        chain = ((((X * b[None, :]) @ S2.T) * m[None, :]) @ S1.T) * a[None, :]
        scale = (np.abs(X) @ b)[:, None] * m.sum() * a[None, :]
        if Y.shape != chain.shape or (np.abs(Y - chain) > 1e-12 * scale).any():
            errs.append(f"DBF chain vs factorisation at {(M, K, Kmid, N)}")
    return errs


def pin_dbf_hadamard(dbf_linear):
    """Closed form: S1 = S2 = H_K, m = c -> W = c K diag(a ⊙ b), so Y = c K X ⊙ (a ⊙ b)."""
    K = 64
    H = sylvester_hadamard(K)
    rng = np.random.default_rng(4)
    a = 2.0 ** rng.integers(-2, 3, size=K)
    b = 2.0 ** rng.integers(-2, 3, size=K)
    c = 0.25
    X = rng.integers(-3, 4, size=(5, K)).astype(np.float64)
    Y = dbf_linear(X, H, H, a, np.full(K, c), b)
    return [] if np.array_equal(Y, c * K * X * (a * b)[None, :]) else ["DBF Hadamard closed form"]


def pin_dbf_int_exact(dbf_linear, seed=23):
    """Integer-exact DBF: fp64 oracle equals an int64 two-stage product."""
    rng = np.random.default_rng(seed)
    M, K, Kmid, N = 4, 96, 64, 48
    X = rng.integers(-1, 2, size=(M, K))
    S2 = random_signs(rng, (Kmid, K)).astype(np.int64)
    S1 = random_signs(rng, (N, Kmid)).astype(np.int64)
    m = rng.integers(1, 4, size=Kmid)
    ea = rng.integers(-1, 3, size=N)
    T1 = (X @ S2.T) * m[None, :]
    Y2 = (T1 @ S1.T) * (2 ** (ea + 1))[None, :]
    Y = dbf_linear(X.astype(np.float64), S1, S2, 2.0 ** ea, m.astype(np.float64), np.ones(K))
    return [] if np.array_equal(Y * 2, Y2.astype(np.float64)) else ["DBF int-exact mismatch"]


def pin_dbf_bruteforce(dbf_linear, seed=29):
    """Pure-Python loops at M=4, K=8, Kmid=6, N=8."""
    rng = np.random.default_rng(seed)
    M, K, Kmid, N = 4, 8, 6, 8
    X = rng.standard_normal((M, K))
    S2 = random_signs(rng, (Kmid, K))
    S1 = random_signs(rng, (N, Kmid))
    b = rng.standard_normal(K)
    m = rng.standard_normal(Kmid)
    a = rng.standard_normal(N)
    Y = dbf_linear(X, S1, S2, a, m, b)
    errs = []
    for i in range(M):
        for j in range(N):
            acc = 0.0
            scale = 0.0
            for l in range(Kmid):
                for k in range(K):
                    t = float(X[i, k]) * float(b[k]) * int(S2[l, k]) * float(m[l]) * int(S1[j, l]) * float(a[j])
                    acc += t
                    scale += abs(t)
            if abs(Y[i, j] - acc) > 1e-13 * scale:
                errs.append(f"DBF brute force ({i},{j})")
    return errs


DBF_PINS = (pin_dbf_chain, pin_dbf_hadamard, pin_dbf_int_exact, pin_dbf_bruteforce)


def pin_backward_finite_differences(onebit_backward, seed=31):
    """The gradients of L = Σ_ij Y_ij dY_ij (Y the OneBit layer) by central
    differences in fp64 (step 1e-6, error O(h^2) plus rounding) must match
    dX, da and db."""
    import oracle as O
    rng = np.random.default_rng(seed)
    M, K, N = 3, 64, 32
    X = rng.standard_normal((M, K))
    S = random_signs(rng, (N, K))
    a = rng.standard_normal(N)
    b = rng.standard_normal(K)
    dY = rng.standard_normal((M, N))
    dX, da, db = onebit_backward(X, S, a, b, dY)

    def L(X_, a_, b_):
        return float((O.onebit_linear(X_, S, a_, b_) * dY).sum())

    h = 1e-6
    errs = []
    for name, base, grad, f in (("dX", X, dX, lambda v: L(v, a, b)),
                                ("da", a, da, lambda v: L(X, v, b)),
                                ("db", b, db, lambda v: L(X, a, v))):
        g = np.asarray(grad, float)
        if g.shape != base.shape:
            errs.append(f"{name} shape {g.shape} != {base.shape}")
            continue
        flat = base.reshape(-1)
        for i in range(0, flat.size, max(1, flat.size // 24)):
            e = np.zeros_like(flat)
            e[i] = h
            num = (f((flat + e).reshape(base.shape)) - f((flat - e).reshape(base.shape))) / (2 * h)
            if abs(num - g.reshape(-1)[i]) > 1e-6 * (1 + abs(num)):
                errs.append(f"{name}[{i}] {g.reshape(-1)[i]} vs finite difference {num}")
    return errs


def pin_backward_bruteforce(onebit_backward, seed=37):
    """Pure-Python loops at M=2, K=8, N=4 over the chain-rule sums."""
    rng = np.random.default_rng(seed)
    M, K, N = 2, 8, 4
    X = rng.standard_normal((M, K))
    S = random_signs(rng, (N, K))
    a = rng.standard_normal(N)
    b = rng.standard_normal(K)
    dY = rng.standard_normal((M, N))
    dX, da, db = onebit_backward(X, S, a, b, dY)
    errs = []
    for i in range(M):
        for k in range(K):
            ref = sum(float(dY[i, j]) * int(S[j, k]) * float(a[j]) * float(b[k]) for j in range(N))
            if abs(dX[i, k] - ref) > 1e-13 * (1 + abs(ref)):
                errs.append(f"dX ({i},{k})")
    for j in range(N):
        ref = sum(float(dY[i, j]) * float(X[i, k]) * int(S[j, k]) * float(b[k]) for i in range(M) for k in range(K))
        if abs(da[j] - ref) > 1e-13 * (1 + abs(ref)):
            errs.append(f"da ({j})")
    for k in range(K):
        ref = sum(float(dY[i, j]) * float(X[i, k]) * int(S[j, k]) * float(a[j]) for i in range(M) for j in range(N))
        if abs(db[k] - ref) > 1e-13 * (1 + abs(ref)):
            errs.append(f"db ({k})")
    return errs


BACKWARD_PINS = (pin_backward_finite_differences, pin_backward_bruteforce)


def pin_layernorm_closed_forms(layernorm_rows):
    """Constant rows normalise to beta; a row of +c / -c in equal numbers to
    ±c / sqrt(c^2 + eps); the affine parameters act elementwise."""
    errs = []
    Y = np.full((2, 8), 3.5)
    if not np.allclose(layernorm_rows(Y, 1e-5), 0.0, atol=0):
        errs.append("constant row not mapped to 0")
    c, eps = 2.0, 1e-3
    Y = np.array([[c, -c] * 4])
    ref = np.array([[1.0, -1.0] * 4]) * c / np.sqrt(c * c + eps)
    if not np.allclose(layernorm_rows(Y, eps), ref, rtol=1e-14, atol=0):
        errs.append("±c row")
    g, bta = np.arange(1.0, 9.0), np.linspace(-1, 1, 8)
    if not np.allclose(layernorm_rows(Y, eps, g, bta), ref * g + bta, rtol=1e-14, atol=1e-15):
        errs.append("affine")
    return errs


def pin_layernorm_invariants_and_bruteforce(layernorm_rows, seed=47):
    """Row mean 0 and mean square var / (var + eps), and pure-Python loops."""
    rng = np.random.default_rng(seed)
    Y = rng.standard_normal((3, 17)) * 5 + 2
    eps = 0.25
    Z = layernorm_rows(Y, eps)
    errs = []
    for i in range(3):
        row = [float(v) for v in Y[i]]
        mu = sum(row) / len(row)
        var = sum((v - mu) ** 2 for v in row) / len(row)
        for j, v in enumerate(row):
            ref = (v - mu) / (var + eps) ** 0.5
            if abs(Z[i, j] - ref) > 1e-13:
                errs.append(f"brute force ({i},{j})")
        if abs(Z[i].mean()) > 1e-13 or abs((Z[i] ** 2).mean() - var / (var + eps)) > 1e-12:
            errs.append(f"invariants row {i}")
    return errs


LAYERNORM_PINS = (pin_layernorm_closed_forms, pin_layernorm_invariants_and_bruteforce)


def run(pins, *fns):
    out = []
    for p in pins:
        try:
            out += [f"{p.__name__}: {e}" for e in p(*fns)]
        except Exception as exc:  # a planted mistake may also raise (shape errors)
            out.append(f"{p.__name__}: raised {type(exc).__name__}: {exc}")
    return out
