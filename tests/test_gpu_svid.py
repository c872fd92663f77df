"""GPU parity of the SVID conversion (obl_svid) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from bit_weight_linear_amd import workloads as WL
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

B = pytest.importorskip("bit_weight_linear_amd.binding", reason="libobl.so not built")


def _rel(x, ref):
    return float(np.max(np.abs(np.asarray(x, float) - ref)) / np.max(np.abs(ref)))


@pytest.mark.parametrize("N,K", [(256, 512), (100, 96), (300, 4128), (11008, 4096)])
@pytest.mark.parametrize("w_dtype,s_dtype", [("f16", "f16"), ("bf16", "f32"), ("f32", "f32")])
def test_svid_matches_oracle(N, K, w_dtype, s_dtype):
    G.say(f"svid N={N} K={K} W {w_dtype} scales {s_dtype}")
    rng = np.random.default_rng(N + K)
    Wd = WL.round_to(rng.standard_normal((N, K)) * 0.02, w_dtype)
    Wd[0, :5] = 0.0                                 # zeros pack as +1
    P, a, b = B.svid(G.dev(Wd, w_dtype), iters=32, scale_dtype=G.TORCH_DT[s_dtype])
    torch.cuda.synchronize()
    S_ref, a_ref, b_ref = O.svid(Wd)
    assert np.array_equal(G.packed_host(P), O.pack_signs(S_ref))
    tol = 2e-5 + (2.0 ** -11 if s_dtype == "f16" else 0.0)
    ea, eb = _rel(G.host64(a), a_ref), _rel(G.host64(b), b_ref)
    G.say(f"  a {ea:.2e} b {eb:.2e}")
    assert ea <= tol and eb <= tol


def test_svid_unaligned_weight_takes_scalar_path():
    """W one element past a 16-byte boundary: the kernels fall back to scalar
    loads and must give the same packing and scales within the tolerance."""
    rng = np.random.default_rng(21)
    N, K = 200, 1024
    Wd = WL.round_to(rng.standard_normal((N, K)) * 0.02, "f16")
    buf = torch.zeros(N * K + 1, dtype=torch.float16, device="cuda")
    buf[1:] = G.dev(Wd, "f16").flatten()
    P, a, b = B.svid(buf[1:].view(N, K), iters=32, scale_dtype=torch.float32)
    torch.cuda.synchronize()
    S_ref, a_ref, b_ref = O.svid(Wd)
    assert np.array_equal(G.packed_host(P), O.pack_signs(S_ref))
    assert _rel(G.host64(a), a_ref) <= 2e-5 and _rel(G.host64(b), b_ref) <= 2e-5


def test_svid_reproducible():
    rng = np.random.default_rng(22)
    Wd = G.dev(WL.round_to(rng.standard_normal((1000, 2048)) * 0.02, "bf16"), "bf16")
    r1 = B.svid(Wd, iters=8, scale_dtype=torch.float32)
    r2 = B.svid(Wd, iters=8, scale_dtype=torch.float32)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def test_svid_recovers_planted_rank1_magnitudes():
    """|W| = a0 b0^T exactly (rank 1): the product a b^T must equal it."""
    rng = np.random.default_rng(3)
    N, K = 192, 320
    a0 = np.abs(rng.standard_normal(N)) + 0.5
    b0 = np.abs(rng.standard_normal(K)) + 0.5
    S = WL.random_signs(rng, (N, K)).astype(np.float64)
    Wd = S * a0[:, None] * b0[None, :]
    P, a, b = B.svid(G.dev(Wd, "f32"), iters=4, scale_dtype=torch.float32)
    torch.cuda.synchronize()
    ab = np.outer(G.host64(a), G.host64(b))
    assert _rel(ab, np.outer(a0, b0)) <= 1e-5
    assert np.array_equal(G.packed_host(P), O.pack_signs(S))


def test_svid_then_linear_is_the_rank1_layer():
    """The converted weight runs through obl_linear: Y = X (W_sign ⊙ a b^T)^T."""
    rng = np.random.default_rng(5)
    N, K, M = 512, 1024, 4
    Wd = WL.round_to(rng.standard_normal((N, K)) * 0.02, "f16")
    P, a, b = B.svid(G.dev(Wd, "f16"), iters=32, scale_dtype=torch.float16)
    X = WL.round_to(rng.standard_normal((M, K)), "bf16")
    Y = B.linear(G.dev(X, "bf16"), P, a, b)
    torch.cuda.synchronize()
    ah, bh = G.host64(a), G.host64(b)
    ref = O.onebit_linear(X, O.sign_pm1(Wd), ah, bh)
    assert O.max_normalised_error(G.host64(Y), ref, O.onebit_error_scale(X, ah, bh)) <= G.TOL_DECODE
