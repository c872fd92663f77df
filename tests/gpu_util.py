"""Helpers for GPU parity tests: move seeded inputs to the device, run the HIP
path through the C ABI, compare with the fp64 oracle at the stated tolerance."""
from __future__ import annotations

import contextlib
import os
import sys

import numpy as np
import torch

import oracle as O

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# Tolerances on the normalised scale |a_j| Σ_k |x_ik b_k| (OneBit) or
# |a_j| Σ_l |m_l| Σ_k |x_ik b_k| (DBF, both stages composed).
TOL_DECODE = 1e-5      # fp32 contraction (M <= 16)
TOL_GEMM = 8e-3        # bf16 matrix-core contraction, bf16 output included (M > 16)
TOL_DBF_GEMM = 1.2e-2  # two bf16 stages: input rounding in each stage + output cast
BF16_U = 2.0 ** -8     # unit roundoff of bf16 (RNE)


def dev(x64, dt: str) -> torch.Tensor:
    """Exact cast of float64 values (representable in dt) to a device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x64)).to(torch.float32).to(TORCH_DT[dt]).cuda()


def signs_dev(S) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(S, dtype=np.int8)).cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def packed_host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def forced_path(path):
    """Force the path (None: the automatic choice) through the library's test-only hook."""
    from bit_weight_linear_amd import binding as B
    return B.forced_kernels(path=path)


def path_of(M: int, path=None) -> str:
    if path:
        return path
    return "lut" if M <= 2 else ("decode" if M <= 16 else "gemm")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_onebit(case, path=None, y_dtype=None):
    from bit_weight_linear_amd import binding as B
    X = dev(case.X, case.x_dtype)
    Wp = B.pack_signs(signs_dev(case.W_sign))
    a = dev(case.a, case.scale_dtype)
    b = dev(case.b, case.scale_dtype)
    yd = y_dtype or case.y_dtype
    with forced_path(path):
        Y = B.linear(X, Wp, a, b, out_dtype=TORCH_DT[yd])
    torch.cuda.synchronize()
    return host64(Y)


def onebit_bound(case, path, y_dtype, Y_ref=None):
    """Per-element allowed |Y - Y_ref|."""
    S = O.onebit_error_scale(case.X, case.a, case.b)
    p = path_of(case.M, path)
    if p == "gemm":
        return TOL_GEMM * S
    bound = TOL_DECODE * S
    if y_dtype == "bf16":
        if Y_ref is None:
            Y_ref = O.onebit_linear(case.X, case.W_sign, case.a, case.b)
        bound = bound + BF16_U * (np.abs(Y_ref) + bound)
    return bound


def check_onebit(case, Y, path=None, y_dtype=None):
    yd = y_dtype or case.y_dtype
    Y_ref = O.onebit_linear(case.X, case.W_sign, case.a, case.b)
    bound = onebit_bound(case, path, yd, Y_ref)
    err = np.abs(Y - Y_ref)
    bad = err > bound
    S = O.onebit_error_scale(case.X, case.a, case.b)
    ratio = O.max_normalised_error(Y, Y_ref, S)
    assert not bad.any(), (f"{case.name} path={path_of(case.M, path)}: {int(bad.sum())} outputs out of "
                           f"tolerance; max normalised error {ratio:.3e}; first at {np.argwhere(bad)[0]}")
    return ratio
