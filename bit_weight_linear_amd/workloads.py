"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws random numbers and rounds them to storage dtypes; it
holds none of the layer's arithmetic.  Every array it returns is float64 (or
int8 for sign matrices) whose values are exactly representable in the storage
dtype named beside it, so the HIP side (after an exact cast) and the fp64
oracle see the same numbers.

Recipes follow the five workloads of the project (shapes of Llama-2-7B /
Llama-3-8B MLP layers, iid +-1 signs, fp16 scales as the DBF page states,
and activations with the outlier structure the LLM.int8() page describes:
a few fixed feature dimensions, six of them, about 60 times larger).  Each
workload uses a fresh ``numpy.random.default_rng(seed)`` (PCG64, seed 0 by
default) and draws tensors in the order they are listed.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` (RNE) and return them as float64.

    bf16 is produced from the fp32 rounding of the value (fp64 -> fp32 RNE,
    then fp32 -> bf16 RNE on the bit pattern).
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        f = np.ascontiguousarray(x.astype(np.float32))
        u = f.view(np.uint32).astype(np.uint64)
        u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
        hi = (u & np.uint64(0xFFFF)).astype(np.uint32) << np.uint32(16)
        return hi.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def random_signs(rng: np.random.Generator, shape) -> np.ndarray:
    """iid +-1 with p = 1/2, as int8."""
    bits = rng.integers(0, 2, size=shape, dtype=np.int8)
    return (1 - 2 * bits).astype(np.int8)


def sylvester_hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), int8 +-1."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    H = np.ones((1, 1), dtype=np.int8)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]]).astype(np.int8)
    return H


@dataclass
class OneBitCase:
    """Inputs of one OneBit layer call ``Y = ((X ⊙ b) W_sign^T) ⊙ a``."""

    name: str
    X: np.ndarray          # [M, K] float64 values, exactly representable in x_dtype
    W_sign: np.ndarray     # [N, K] int8 +-1
    a: np.ndarray          # [N] float64 values in scale_dtype
    b: np.ndarray          # [K] float64 values in scale_dtype
    x_dtype: str
    scale_dtype: str
    y_dtype: str
    meta: Dict = field(default_factory=dict)

    @property
    def M(self):
        return self.X.shape[0]

    @property
    def K(self):
        return self.X.shape[1]

    @property
    def N(self):
        return self.W_sign.shape[0]


@dataclass
class DBFCase:
    """Inputs of one DBF call ``Y = ((((X ⊙ b) S2^T) ⊙ m) S1^T) ⊙ a``."""

    name: str
    X: np.ndarray          # [M, K]
    S2: np.ndarray         # [Kmid, K] int8 +-1
    S1: np.ndarray         # [N, Kmid] int8 +-1
    b: np.ndarray          # [K]
    m: np.ndarray          # [Kmid]
    a: np.ndarray          # [N]
    x_dtype: str
    scale_dtype: str
    y_dtype: str
    meta: Dict = field(default_factory=dict)

    @property
    def M(self):
        return self.X.shape[0]

    @property
    def K(self):
        return self.X.shape[1]

    @property
    def Kmid(self):
        return self.S2.shape[0]

    @property
    def N(self):
        return self.S1.shape[0]


def _abs_normal(rng, std, size, eps):
    return np.abs(rng.normal(0.0, std, size=size)) + eps


def _activations(rng, M, K, outliers: int, factor: float):
    X = rng.standard_normal((M, K))
    ch = None
    if outliers:
        ch = np.sort(rng.choice(K, outliers, replace=False))
        X[:, ch] *= factor       # scaled in fp64, rounded once afterwards
    return X, ch


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------
WORKLOADS = {
    1: "onebit-tiny-4x512x512-f32",
    2: "llama7b-mlp-decode-gemv-1x4096x11008",
    3: "batched-decode-16x4096x4096",
    4: "prefill-gemm-2048x4096x14336",
    5: "dbf-1.5bit-8x4096-3072-4096",
}


def workload(i: int, seed: int = 0):
    """Workload ``i`` (1..5) drawn from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    if i == 1:
        X = rng.standard_normal((4, 512))
        W = random_signs(rng, (512, 512))
        a = _abs_normal(rng, 1.0, 512, 0.1)
        b = _abs_normal(rng, 1.0, 512, 0.1)
        return OneBitCase(WORKLOADS[1], round_to(X, "f32"), W, round_to(a, "f32"),
                          round_to(b, "f32"), "f32", "f32", "f32")
    if i in (2, 3):
        M, N = (1, 11008) if i == 2 else (16, 4096)
        K = 4096
        X, ch = _activations(rng, M, K, 6, 60.0)
        W = random_signs(rng, (N, K))
        a = _abs_normal(rng, 0.02, N, 1e-3)
        b = _abs_normal(rng, 0.02, K, 1e-3)
        return OneBitCase(WORKLOADS[i], round_to(X, "bf16"), W, round_to(a, "f16"),
                          round_to(b, "f16"), "bf16", "f16", "f32",
                          meta={"outlier_channels": ch.tolist()})
    if i == 4:
        M, K, N = 2048, 4096, 14336
        X = rng.standard_normal((M, K))
        W = random_signs(rng, (N, K))
        a = _abs_normal(rng, 0.02, N, 1e-3)
        b = _abs_normal(rng, 0.02, K, 1e-3)
        return OneBitCase(WORKLOADS[4], round_to(X, "bf16"), W, round_to(a, "f16"),
                          round_to(b, "f16"), "bf16", "f16", "bf16")
    if i == 5:
        M, K, Kmid, N = 8, 4096, 3072, 4096
        X = rng.standard_normal((M, K))
        S2 = random_signs(rng, (Kmid, K))
        S1 = random_signs(rng, (N, Kmid))
        b = _abs_normal(rng, 1.0, K, 0.1)
        m = _abs_normal(rng, 1.0, Kmid, 0.1)
        a = _abs_normal(rng, 1.0, N, 0.1)
        return DBFCase(WORKLOADS[5], round_to(X, "bf16"), S2, S1, round_to(b, "f16"),
                       round_to(m, "f16"), round_to(a, "f16"), "bf16", "f16", "f32")
    raise ValueError("workload index must be 1..5")


# --------------------------------------------------------------------------
# Generic cases for parity sweeps and edge cases
# --------------------------------------------------------------------------
def onebit_case(M: int, K: int, N: int, x_dtype="bf16", scale_dtype="f16", y_dtype="f32",
                seed: int = 0, kind: str = "normal", scale_std: Optional[float] = None,
                name: Optional[str] = None) -> OneBitCase:
    """A OneBit call of any shape.

    ``kind``:
      * ``"normal"``  -- X ~ N(0,1) (six x60 outlier columns when K >= 64), scales
        ~ |N(0, std)| + eps (std 0.02 for fp16 scales, 1.0 for fp32);
      * ``"int_exact"`` -- X in {-2..2}, a and b in {1/2, 1, 2, 4}: every partial
        sum of x·b is a multiple of 1/2 of size at most 8K, i.e. below 2^24
        halves for K < 2^20, so any summation order gives the same fp32 result;
      * ``"signed_scales"`` -- as normal but a and b take random signs.
    """
    rng = np.random.default_rng(seed)
    if kind == "int_exact":
        X = rng.integers(-2, 3, size=(M, K)).astype(np.float64)
        W = random_signs(rng, (N, K))
        pw = np.array([0.5, 1.0, 2.0, 4.0])
        a = pw[rng.integers(0, 4, size=N)]
        b = pw[rng.integers(0, 4, size=K)]
    else:
        outl = 6 if K >= 64 else 0
        X, _ = _activations(rng, M, K, outl, 60.0)
        W = random_signs(rng, (N, K))
        std = scale_std if scale_std is not None else (1.0 if scale_dtype == "f32" else 0.02)
        eps = 0.1 if std >= 1.0 else 1e-3
        a = _abs_normal(rng, std, N, eps)
        b = _abs_normal(rng, std, K, eps)
        if kind == "signed_scales":
            a = a * np.where(rng.integers(0, 2, N) == 1, -1.0, 1.0)
            b = b * np.where(rng.integers(0, 2, K) == 1, -1.0, 1.0)
        elif kind != "normal":
            raise ValueError(f"unknown kind {kind!r}")
    return OneBitCase(name or f"onebit-{kind}-{M}x{K}x{N}", round_to(X, x_dtype), W,
                      round_to(a, scale_dtype), round_to(b, scale_dtype),
                      x_dtype, scale_dtype, y_dtype)


def dbf_case(M: int, K: int, Kmid: int, N: int, x_dtype="bf16", scale_dtype="f16",
             y_dtype="f32", seed: int = 0, kind: str = "normal",
             name: Optional[str] = None) -> DBFCase:
    """A DBF call of any shape.  ``kind="int_exact"``: X in {-1,0,1}, b = m = 1,
    a in {1/2,1,2,4}, so T1 holds integers with |T1| <= K and every partial sum
    of T1 S1^T is an integer of size at most K·Kmid, exact in fp32 for
    K·Kmid < 2^24; the final scaling by a power of two is exact."""
    rng = np.random.default_rng(seed)
    if kind == "int_exact":
        X = rng.integers(-1, 2, size=(M, K)).astype(np.float64)
        S2 = random_signs(rng, (Kmid, K))
        S1 = random_signs(rng, (N, Kmid))
        b = np.ones(K)
        m = np.ones(Kmid)
        a = np.array([0.5, 1.0, 2.0, 4.0])[rng.integers(0, 4, size=N)]
    elif kind == "normal":
        X = rng.standard_normal((M, K))
        S2 = random_signs(rng, (Kmid, K))
        S1 = random_signs(rng, (N, Kmid))
        b = _abs_normal(rng, 1.0, K, 0.1)
        m = _abs_normal(rng, 1.0, Kmid, 0.1)
        a = _abs_normal(rng, 1.0, N, 0.1)
    else:
        raise ValueError(f"unknown kind {kind!r}")
    return DBFCase(name or f"dbf-{kind}-{M}x{K}x{Kmid}x{N}", round_to(X, x_dtype), S2, S1,
                   round_to(b, scale_dtype), round_to(m, scale_dtype), round_to(a, scale_dtype),
                   x_dtype, scale_dtype, y_dtype)
