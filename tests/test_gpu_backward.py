"""GPU parity of the transposed sign packing and of the layer's backward
(obl_transpose_signs, obl_linear_backward) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from bit_weight_linear_amd import workloads as WL
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

B = pytest.importorskip("bit_weight_linear_amd.binding", reason="libobl.so not built")


@pytest.mark.parametrize("rows,K", [(32, 32), (64, 128), (96, 160), (4096, 4096), (11008, 4096), (160, 11008)])
def test_transpose_signs_bit_exact(rows, K):
    G.say(f"transpose rows={rows} K={K}")
    rng = np.random.default_rng(rows + K)
    S = WL.random_signs(rng, (rows, K))
    P = B.pack_signs(G.signs_dev(S))
    PT = B.transpose_signs(P, rows, K)
    torch.cuda.synchronize()
    assert np.array_equal(G.packed_host(PT), O.transpose_signs(O.pack_signs(S), rows, K))
    # transposing back restores the packing
    assert torch.equal(B.transpose_signs(PT, K, rows), P)


def _case(M, K, N, x_dtype, scale_dtype, seed):
    rng = np.random.default_rng(seed)
    X = WL.round_to(rng.standard_normal((M, K)), x_dtype)
    dY = WL.round_to(rng.standard_normal((M, N)), x_dtype)
    S = WL.random_signs(rng, (N, K))
    a = WL.round_to(np.abs(rng.standard_normal(N)) * 0.05 + 1e-3, scale_dtype)
    b = WL.round_to(np.abs(rng.standard_normal(K)) + 0.1, scale_dtype)
    return X, dY, S, a, b


def _run(X, dY, S, a, b, x_dtype, scale_dtype, dx_dtype):
    W = B.pack_signs(G.signs_dev(S))
    Wt = B.transpose_signs(W, S.shape[0], S.shape[1])
    dX, da, db, ws = B.linear_backward(G.dev(dY, x_dtype), G.dev(X, x_dtype), W, Wt, G.dev(a, scale_dtype),
                                       G.dev(b, scale_dtype), dx_dtype=G.TORCH_DT[dx_dtype])
    torch.cuda.synchronize()
    return G.host64(dX), G.host64(da), G.host64(db), ws


# (5, 1024, 512), (16, 4096, 4096), (17, 4096, 512) and (24, 1152, 640) with bf16
# inputs run both contractions on the whole-K decode kernel, whose epilogue
# forms dX, da and db; (9, 544, 96) and fp32 inputs take the reduction kernel.
@pytest.mark.parametrize("M,K,N", [(1, 512, 256), (2, 4096, 1024), (5, 1024, 512), (16, 4096, 4096),
                                   (9, 544, 96), (64, 1024, 1024), (300, 512, 768), (17, 4096, 512),
                                   (24, 1152, 640)])
@pytest.mark.parametrize("dts", [("bf16", "f16", "f32"), ("f32", "f32", "f32"), ("bf16", "f16", "bf16")],
                         ids=lambda d: "-".join(d))
def test_backward_parity(M, K, N, dts):
    x_dtype, scale_dtype, dx_dtype = dts
    G.say(f"backward M={M} K={K} N={N} {dts}")
    X, dY, S, a, b = _case(M, K, N, x_dtype, scale_dtype, seed=M + K + N)
    dX, da, db, ws = _run(X, dY, S, a, b, x_dtype, scale_dtype, dx_dtype)
    rdX, rda, rdb = O.onebit_backward(X, S, a, b, dY)
    sdx, sda, sdb = O.backward_error_scales(X, a, b, dY)
    tol = G.TOL_DECODE if M <= 16 else G.TOL_GEMM
    tol_dx = tol + (G.BF16_U if dx_dtype == "bf16" else 0.0)
    e = (O.max_normalised_error(dX, rdX, sdx), O.max_normalised_error(da, rda, sda),
         O.max_normalised_error(db, rdb, sdb))
    G.say(f"  dX {e[0]:.2e} da {e[1]:.2e} db {e[2]:.2e}")
    assert e[0] <= tol_dx and e[1] <= tol and e[2] <= tol
    # the workspace holds T = (X ⊙ b) W^T [M][N], then U = (dY ⊙ a) W [M][K]
    T = G.host64(ws[: M * N].view(M, N))
    assert O.max_normalised_error(T, O.onebit_linear(X, S, np.ones(N), b),
                                  O.onebit_error_scale(X, np.ones(N), b)) <= tol


def test_backward_integer_exact_bitwise():
    """Integer-valued inputs with power-of-two scales: every partial sum is an
    exactly representable integer multiple of a power of two, so all paths
    must agree with the oracle bit for bit (decode sizes)."""
    rng = np.random.default_rng(7)
    for M in (1, 4, 16):
        K, N = 1024, 512
        X = rng.integers(-2, 3, size=(M, K)).astype(np.float64)
        dY = rng.integers(-2, 3, size=(M, N)).astype(np.float64)
        S = WL.random_signs(rng, (N, K))
        a = 2.0 ** rng.integers(-1, 3, size=N)
        b = 2.0 ** rng.integers(-1, 3, size=K)
        dX, da, db, _ = _run(X, dY, S, a, b, "bf16", "f16", "f32")
        rdX, rda, rdb = O.onebit_backward(X, S, a, b, dY)
        assert np.array_equal(dX, rdX) and np.array_equal(da, rda) and np.array_equal(db, rdb)


def test_backward_m0_writes_zero_scale_gradients():
    K, N = 256, 128
    S = WL.random_signs(np.random.default_rng(3), (N, K))
    W = B.pack_signs(G.signs_dev(S))
    Wt = B.transpose_signs(W, N, K)
    X = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, N), dtype=torch.bfloat16, device="cuda")
    one = lambda n: torch.ones(n, dtype=torch.float16, device="cuda")
    dX, da, db, _ = B.linear_backward(dY, X, W, Wt, one(N), one(K), workspace=torch.empty(1, device="cuda"))
    torch.cuda.synchronize()
    assert dX.shape == (0, K) and torch.count_nonzero(da) == 0 and torch.count_nonzero(db) == 0


def test_backward_reproducible():
    X, dY, S, a, b = _case(16, 4096, 1024, "bf16", "f16", seed=5)
    r1 = _run(X, dY, S, a, b, "bf16", "f16", "f32")
    r2 = _run(X, dY, S, a, b, "bf16", "f16", "f32")
    for u, v in zip(r1[:3], r2[:3]):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("impl", ["wk1", "wk2", "wk4"])
def test_backward_fused_epilogue_column_groups(impl, forcer):
    """The gradient epilogue at every column count per wave (16, 32 and 64
    columns per workgroup), dX in bf16, against the oracle."""
    forcer(decode=impl)
    M, K, N = 16, 1024, 2048
    X, dY, S, a, b = _case(M, K, N, "bf16", "f16", seed=41)
    dX, da, db, _ = _run(X, dY, S, a, b, "bf16", "f16", "bf16")
    rdX, rda, rdb = O.onebit_backward(X, S, a, b, dY)
    sdx, sda, sdb = O.backward_error_scales(X, a, b, dY)
    assert O.max_normalised_error(dX, rdX, sdx) <= G.TOL_DECODE + G.BF16_U
    assert O.max_normalised_error(da, rda, sda) <= G.TOL_DECODE
    assert O.max_normalised_error(db, rdb, sdb) <= G.TOL_DECODE


# Shapes whose two contractions share one whole-K kernel instance run as one
# launch: square and oblong layers, 17..32 rows (four waves), and K = 32768
# against N = 4096 (the two contractions need different instances: two
# launches).  With the column groups per wave forced, one launch and two run
# the same workgroups and must agree bitwise; by default the pair picks its
# own column count (both grids within one workgroup per CU), which changes the
# order of the fp32 adds, so it is held to the oracle's bound.
PAIR_CASES = [(16, 4096, 4096), (5, 1024, 512), (8, 2048, 4096), (3, 4096, 11008), (24, 1152, 640),
              (32, 4096, 4096), (4, 32768, 4096)]


def _oracle_bounds(X, dY, S, a, b, got, dx_dtype):
    rdX, rda, rdb = O.onebit_backward(X, S, a, b, dY)
    sdx, sda, sdb = O.backward_error_scales(X, a, b, dY)
    tol_dx = G.TOL_DECODE + (G.BF16_U if dx_dtype == "bf16" else 0.0)
    assert O.max_normalised_error(got[0], rdX, sdx) <= tol_dx
    assert O.max_normalised_error(got[1], rda, sda) <= G.TOL_DECODE
    assert O.max_normalised_error(got[2], rdb, sdb) <= G.TOL_DECODE


@pytest.mark.parametrize("M,K,N", PAIR_CASES)
@pytest.mark.parametrize("impl", ["wk1", "wk2"])
def test_backward_one_launch_equals_two(M, K, N, impl, forcer):
    """Same column groups per wave: the one-launch backward gives bitwise the
    dX, da, db and workspace of two launches."""
    forcer(decode=impl)
    G.say(f"backward one vs two launches M={M} K={K} N={N} {impl}")
    X, dY, S, a, b = _case(M, K, N, "bf16", "f16", seed=M * 3 + K + N)
    one = _run(X, dY, S, a, b, "bf16", "f16", "f32")
    with B.forced_kernels(pair="off"):
        two = _run(X, dY, S, a, b, "bf16", "f16", "f32")
    for u, v, what in zip(one[:3], two[:3], ("dX", "da", "db")):
        assert np.array_equal(u, v), f"{what} differs between one and two launches"
    assert torch.equal(one[3], two[3]), "workspace differs between one and two launches"
    _oracle_bounds(X, dY, S, a, b, one, "f32")


@pytest.mark.parametrize("M,K,N", PAIR_CASES)
@pytest.mark.parametrize("dx_dtype", ["f32", "bf16"])
def test_backward_default_pairing_against_oracle(M, K, N, dx_dtype):
    G.say(f"backward default pairing M={M} K={K} N={N} dX {dx_dtype}")
    X, dY, S, a, b = _case(M, K, N, "bf16", "f16", seed=M * 5 + K + N)
    _oracle_bounds(X, dY, S, a, b, _run(X, dY, S, a, b, "bf16", "f16", dx_dtype), dx_dtype)
