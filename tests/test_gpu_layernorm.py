"""GPU parity of the LayerNorm after the layer (obl_layernorm,
obl_linear_layernorm) against the fp64 oracle.

Tolerances, from the kernel's fp32 arithmetic: each row sum adds at most ~300
terms in sequence here (per-thread chunks, up to 274 on the longest scalar
rows tested, then the wave tree and the waves), so the mean is off by at most
~300·2^-24·mean|y| and the standard deviation by a few hundred ulps relative;
on the normalised output that is below 2e-5·(mean|y| / s + |ẑ|) with
s = sqrt(σ² + eps).  The layer's own error
|δY_ij| <= tol·|a_j| Σ_k |x_ik b_k| moves ẑ by at most
(|δY_ij| + max_j |δY_ij| · (1 + |ẑ_ij|)) / s (mean and spread are both
1-Lipschitz in the max norm)."""
import numpy as np
import pytest
import torch

import oracle as O
from bit_weight_linear_amd import workloads as WL
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

B = pytest.importorskip("bit_weight_linear_amd.binding", reason="libobl.so not built")

LN_REL = 2e-5


def _stats(Y, eps):
    mu = Y.mean(1, keepdims=True)
    s = np.sqrt(((Y - mu) ** 2).mean(1, keepdims=True) + eps)
    return mu, s


def ln_bound(Y, eps, gamma, beta, z_dtype, dY=None):
    """Allowed |Z - Z_ref| per element; dY = per-element bound on the input's own error."""
    mu, s = _stats(Y, eps)
    zhat = (Y - mu) / s
    g = np.ones(Y.shape[1]) if gamma is None else np.abs(gamma)
    bt = np.zeros(Y.shape[1]) if beta is None else np.abs(beta)
    bound = LN_REL * (np.abs(Y).mean(1, keepdims=True) / s + np.abs(zhat)) * g[None, :]
    bound = bound + 2e-6 * (np.abs(zhat) * g[None, :] + bt[None, :])
    if dY is not None:
        dmax = dY.max(1, keepdims=True)
        bound = bound + 1.1 * (dY + dmax * (1 + np.abs(zhat))) / s * g[None, :]
    if z_dtype == "bf16":
        zref = O.layernorm_rows(Y, eps, gamma, beta)
        bound = bound + G.BF16_U * (np.abs(zref) + bound)
    return bound


def _check(Z, Zref, bound, what):
    err = np.abs(Z - Zref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs out of tolerance, first at "
                           f"{np.argwhere(bad)[0]}, err/bound max {float(np.max(err / bound)):.3g}")


def _affine(rng, N, kind, dt):
    if kind == "none":
        return None, None
    g = WL.round_to(rng.standard_normal(N) * 0.5 + 1.0, dt)
    bt = WL.round_to(rng.standard_normal(N) * 0.1, dt)
    return (g, bt) if kind == "both" else (None, bt)


# Every kernel variant: 1024-thread register path with 4 and 8 chunks (M < 256),
# 256-thread with 4 and 8 chunks, 512-thread with 8 (rows of 2 K..4 K vectors,
# (300, 14336) and (270, 9000)), the vector window path (rows too long
# for registers) and the scalar window path (N % 4 != 0), plus tiny rows.
SHAPES = [(1, 11008), (4, 4096), (3, 1000), (16, 14336), (3, 20000), (256, 4096), (260, 8000),
          (300, 14336), (270, 9000), (257, 4097), (2, 70000), (300, 70001), (5, 1), (2, 3), (1, 64)]


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("y_dtype,z_dtype", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
@pytest.mark.parametrize("affine", ["none", "both", "beta"])
def test_layernorm_matches_oracle(M, N, y_dtype, z_dtype, affine):
    G.say(f"layernorm M={M} N={N} y {y_dtype} z {z_dtype} affine {affine}")
    rng = np.random.default_rng(M * 7 + N)
    Y = WL.round_to(rng.standard_normal((M, N)) * 2.0 + 3.0, y_dtype)
    gdt = "f16" if affine == "beta" else "f32"
    gamma, beta = _affine(rng, N, affine, gdt)
    eps = 1e-5
    Z = B.layernorm(G.dev(Y, y_dtype), eps,
                    None if gamma is None else G.dev(gamma, gdt), None if beta is None else G.dev(beta, gdt),
                    out_dtype=G.TORCH_DT[z_dtype])
    torch.cuda.synchronize()
    Zref = O.layernorm_rows(Y, eps, gamma, beta)
    _check(G.host64(Z), Zref, ln_bound(Y, eps, gamma, beta, z_dtype), f"M={M} N={N}")


def test_layernorm_degenerate_rows():
    """Constant rows (exact mean) give exactly beta; N = 1 gives beta; a large
    epsilon shrinks the output as the formula says."""
    N = 4096
    Y = np.full((3, N), 3.0)
    Y[1] = -0.5
    Y[2] = 0.0
    beta = WL.round_to(np.linspace(-1, 1, N), "f32")
    Z = B.layernorm(G.dev(Y, "f32"), 1e-5, None, G.dev(beta, "f32"))
    torch.cuda.synchronize()
    assert np.array_equal(G.host64(Z), np.tile(beta, (3, 1)))
    Z1 = B.layernorm(G.dev(np.array([[5.0], [-2.0]]), "f32"), 1e-5)
    torch.cuda.synchronize()
    assert np.array_equal(G.host64(Z1), np.zeros((2, 1)))
    Yb = np.array([[1.0, -1.0] * 512])
    Zb = B.layernorm(G.dev(Yb, "f32"), 3.0)
    torch.cuda.synchronize()
    assert np.allclose(G.host64(Zb), Yb / 2.0, rtol=1e-6, atol=0)


def test_layernorm_unaligned_affine_takes_scalar_path():
    """gamma / beta one element past an 8-byte boundary: the vector path is not
    allowed, the scalar window path must give the same values."""
    rng = np.random.default_rng(4)
    M, N = 3, 4096
    Y = rng.standard_normal((M, N))
    gamma = WL.round_to(rng.standard_normal(N) + 1, "f16")
    beta = WL.round_to(rng.standard_normal(N) * 0.1, "f16")
    gbuf = torch.zeros(N + 1, dtype=torch.float16, device="cuda")
    bbuf = torch.zeros(N + 1, dtype=torch.float16, device="cuda")
    gbuf[1:] = G.dev(gamma, "f16")
    bbuf[1:] = G.dev(beta, "f16")
    Yd = G.dev(Y, "f32")
    Z = B.layernorm(Yd, 1e-5, gbuf[1:], bbuf[1:])
    Za = B.layernorm(Yd, 1e-5, G.dev(gamma, "f16"), G.dev(beta, "f16"))
    torch.cuda.synchronize()
    Zref = O.layernorm_rows(Y, 1e-5, gamma, beta)
    bound = ln_bound(Y, 1e-5, gamma, beta, "f32")
    _check(G.host64(Z), Zref, bound, "unaligned affine")
    _check(G.host64(Za), Zref, bound, "aligned affine")


def test_layernorm_reproducible_and_m0():
    rng = np.random.default_rng(9)
    Yd = G.dev(rng.standard_normal((64, 14336)), "f32")
    z1 = B.layernorm(Yd)
    z2 = B.layernorm(Yd)
    torch.cuda.synchronize()
    assert torch.equal(z1, z2)
    z0 = B.layernorm(torch.empty((0, 128), device="cuda"))
    torch.cuda.synchronize()
    assert z0.shape == (0, 128)


LIN_CASES = [(1, 4096, 11008), (2, 1024, 512), (4, 4096, 4096), (16, 4096, 11008), (9, 544, 96),
             (64, 1024, 1024), (300, 512, 768)]


@pytest.mark.parametrize("M,K,N", LIN_CASES)
@pytest.mark.parametrize("z_dtype,affine", [("f32", "none"), ("bf16", "both")])
def test_linear_layernorm_matches_oracle(M, K, N, z_dtype, affine):
    G.say(f"linear+layernorm M={M} K={K} N={N} z {z_dtype} affine {affine}")
    c = WL.onebit_case(M, K, N, seed=M + K + N)
    rng = np.random.default_rng(N)
    gamma, beta = _affine(rng, N, affine, c.scale_dtype)
    dv = lambda v: None if v is None else G.dev(v, c.scale_dtype)
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    Z, ws = B.linear_layernorm(G.dev(c.X, c.x_dtype), Wp, G.dev(c.a, c.scale_dtype), G.dev(c.b, c.scale_dtype),
                               1e-5, dv(gamma), dv(beta), out_dtype=G.TORCH_DT[z_dtype])
    torch.cuda.synchronize()
    Yref = O.onebit_linear(c.X, c.W_sign, c.a, c.b)
    tol = G.TOL_DECODE if M <= 16 else G.TOL_GEMM
    dY = tol * O.onebit_error_scale(c.X, c.a, c.b)
    # the workspace holds the layer output Y in fp32
    _check(G.host64(ws), Yref, dY, "workspace Y")
    _check(G.host64(Z), O.layernorm_rows(Yref, 1e-5, gamma, beta),
           ln_bound(Yref, 1e-5, gamma, beta, z_dtype, dY), f"Z M={M} K={K} N={N}")


def test_linear_layernorm_full_prefill_sampled_rows():
    """M = 2048, K = 4096, N = 14336 through the prefill kernel; LayerNorm is
    row-local, so the oracle computes the sampled rows alone."""
    M, K, N = 2048, 4096, 14336
    G.say(f"linear+layernorm full size {M}x{K}x{N}")
    c = WL.onebit_case(M, K, N, seed=11)
    rng = np.random.default_rng(12)
    gamma, beta = _affine(rng, N, "both", c.scale_dtype)
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    Z, ws = B.linear_layernorm(G.dev(c.X, c.x_dtype), Wp, G.dev(c.a, c.scale_dtype), G.dev(c.b, c.scale_dtype),
                               1e-5, G.dev(gamma, c.scale_dtype), G.dev(beta, c.scale_dtype),
                               out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.choice(M, 6, replace=False), [0, M - 1]]))
    Yref = O.onebit_linear(c.X[rows], c.W_sign, c.a, c.b)
    dY = G.TOL_GEMM * O.onebit_error_scale(c.X[rows], c.a, c.b)
    _check(G.host64(ws[torch.from_numpy(rows).cuda()]), Yref, dY, "workspace Y")
    _check(G.host64(Z[torch.from_numpy(rows).cuda()]), O.layernorm_rows(Yref, 1e-5, gamma, beta),
           ln_bound(Yref, 1e-5, gamma, beta, "bf16", dY), "Z sampled rows")
