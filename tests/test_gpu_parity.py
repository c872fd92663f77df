"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (normalised scale S_ij = |a_j| Σ_k |x_ik b_k|):
  * M <= 16 (LUT GEMV and decode kernel): 1e-5 · S (fp32 contraction), plus
    one bf16 rounding of the output (2^-8 relative) when Y is bf16;
  * M > 16 (bf16 matrix-core GEMM): 8e-3 · S, output cast included.
Exact regimes (integer-exact inputs, Hadamard, the LLM.int8() page example)
require bit-exact equality on every path.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from bit_weight_linear_amd import workloads as WL
from tests import gpu_util as G
from tests.oracle_pins import GOLDEN, fwht_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from bit_weight_linear_amd import binding as B  # noqa: E402  (loads libobl.so)


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("rows,K", [(1, 32), (3, 96), (7, 4096), (512, 512), (4096, 3072)])
@pytest.mark.parametrize("dt", ["i8", "f32", "f16", "bf16"])
def test_pack_bit_exact(rows, K, dt):
    G.say(f"pack {dt} {rows}x{K}")
    rng = np.random.default_rng(rows * 7 + K)
    S = rng.standard_normal((rows, K))
    S[rng.random((rows, K)) < 0.05] = 0.0
    S[rng.random((rows, K)) < 0.05] = -0.0
    if dt == "i8":
        S = WL.random_signs(rng, (rows, K))
        t = G.signs_dev(S)
    else:
        S = WL.round_to(S, dt)
        t = torch.from_numpy(S).to(torch.float32).to(G.TORCH_DT[dt]).cuda()  # keeps -0.0
    P = B.pack_signs(t)
    torch.cuda.synchronize()
    assert np.array_equal(G.packed_host(P), O.pack_signs(S))


def test_pack_largest_config_shape():
    rng = np.random.default_rng(4)
    S = WL.random_signs(rng, (14336, 4096))
    P = B.pack_signs(G.signs_dev(S))
    assert np.array_equal(G.packed_host(P), O.pack_signs(S))


# ------------------------------------------------------------------ parity sweeps per path
LUT_CASES = [
    (1, 32, 1), (1, 96, 33), (2, 128, 257), (1, 4128, 300), (2, 8192, 200), (1, 4096, 4099),
    (2, 544, 130), (1, 4096, 17), (1, 128, 64), (1, 2048, 513), (1, 3968, 100),
]
DTYPE_COMBOS = [("bf16", "f16", "f32"), ("f32", "f32", "f32"), ("bf16", "f16", "bf16"),
                ("f32", "f16", "f32")]


@pytest.mark.parametrize("M,K,N", LUT_CASES)
@pytest.mark.parametrize("dts", DTYPE_COMBOS, ids=lambda d: "-".join(d))
def test_lut_path(M, K, N, dts):
    G.say(f"lut M={M} K={K} N={N} {dts}")
    c = WL.onebit_case(M, K, N, *dts, seed=M + K + N)
    G.check_onebit(c, G.run_onebit(c, "lut"), "lut")


DECODE_CASES = [
    (1, 32, 17), (3, 512, 64), (5, 544, 100), (8, 1024, 1000), (16, 4096, 4096), (16, 96, 33),
    (2, 4096, 4096), (11, 8192, 129), (4, 512, 512),
]


@pytest.mark.parametrize("M,K,N", DECODE_CASES)
@pytest.mark.parametrize("dts", DTYPE_COMBOS, ids=lambda d: "-".join(d))
def test_decode_path(M, K, N, dts):
    G.say(f"decode M={M} K={K} N={N} {dts}")
    c = WL.onebit_case(M, K, N, *dts, seed=M * 3 + K + N)
    G.check_onebit(c, G.run_onebit(c, "decode"), "decode")


# Small grids split K (bf16 x, K % 128 == 0): (256, 4096, 224) and (600, 4096, 449)
# into 8 slices, (300, 1152, 672) into 2, (40, 2048, 98) into 4 with N % 4 != 0
# (scalar partials and reduction), (200, 4736, 1000) into 8 uneven slices (37
# stages of 128 k); (255, 512, 448) has too few stages to split.  K = 128,
# 256 and 640 run 1, 2 and 5 stages whole (the stage loop is unrolled by three;
# the last stage also reads a clamped next stage).
GEMM_CASES = [
    (17, 32, 16), (64, 96, 225), (255, 512, 448), (256, 4096, 224), (257, 160, 1000),
    (600, 4096, 449), (33, 64, 33), (513, 384, 230), (300, 1152, 672), (40, 2048, 98),
    (200, 4736, 1000), (130, 128, 500), (70, 256, 257), (129, 640, 449),
]
GEMM_DTYPES = [("bf16", "f16", "bf16"), ("bf16", "f16", "f32"), ("bf16", "f32", "bf16"),
               ("f32", "f32", "f32"), ("f32", "f16", "bf16")]


@pytest.mark.parametrize("M,K,N", GEMM_CASES)
@pytest.mark.parametrize("dts", GEMM_DTYPES, ids=lambda d: "-".join(d))
@pytest.mark.parametrize("impl", ["auto", "w7", "w4", "w2", "w1", "v2", "v1"])
def test_gemm_path(M, K, N, dts, impl, forcer):
    """impl=auto picks the main 32x32 kernel where it applies (K % 128 == 0;
    fp32 or misaligned x through the prescale pass) and its tile; w7 / w4 / w2
    force the 128-row tiles of 448 / 256 / 128 columns, w1 the 64 x 128 tile,
    v2 the LDS-staged 16x16 kernel, v1 the 8-wave kernel."""
    if impl != "auto":
        forcer(gemm=impl)
    G.say(f"gemm[{impl}] M={M} K={K} N={N} {dts}")
    c = WL.onebit_case(M, K, N, *dts, seed=M + 2 * K + N)
    G.check_onebit(c, G.run_onebit(c, "gemm"), "gemm")


@pytest.mark.parametrize("path,M", [("lut", 1), ("lut", 2), ("decode", 7), ("gemm", 40)])
def test_signed_scales(path, M):
    G.say(f"signed scales {path} M={M}")
    c = WL.onebit_case(M, 512, 96, kind="signed_scales", seed=99)
    G.check_onebit(c, G.run_onebit(c, path), path)


def test_gemm_misaligned_activations_use_convert_mode():
    """X starting at an odd bf16 element (2-byte aligned only) must still be right."""
    G.say("gemm misaligned X")
    c = WL.onebit_case(48, 256, 96, seed=5)
    flat = torch.zeros(48 * 256 + 1, dtype=torch.bfloat16, device="cuda")
    X = flat[1:].view(48, 256)
    X.copy_(G.dev(c.X, "bf16"))
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    Y = B.linear(X, Wp, G.dev(c.a, "f16"), G.dev(c.b, "f16"))
    G.check_onebit(c, G.host64(Y), "gemm")


# ------------------------------------------------------------------ the five workloads
def test_workload1_tiny_f32():
    c = WL.workload(1)
    G.say(c.name)
    r = G.check_onebit(c, G.run_onebit(c))
    G.say(f"  max normalised error {r:.3e}")


def test_workload2_decode_gemv():
    c = WL.workload(2)
    G.say(c.name)
    r = G.check_onebit(c, G.run_onebit(c))
    G.say(f"  max normalised error {r:.3e}")


def test_workload3_batched_decode():
    c = WL.workload(3)
    G.say(c.name)
    r = G.check_onebit(c, G.run_onebit(c))
    G.say(f"  max normalised error {r:.3e}")


def test_workload4_prefill_full():
    """The full 2048 x 4096 x 14336 launch (bf16 output, the kernel and tile the
    bench times) against the fp64 oracle on every one of its 29.4 M outputs, at
    the prefill tolerance on the normalised scale."""
    c = WL.workload(4)
    G.say(c.name)
    Y = G.run_onebit(c)
    assert np.isfinite(Y).all()
    r = G.check_onebit(c, Y)
    G.say(f"  max normalised error over all {Y.size} outputs {r:.3e}")


def test_workload4_shape_integer_exact_bf16():
    """Integer-exact inputs at exactly the workload-4 shape through the default
    prefill kernel with bf16 output: every partial sum is exact in fp32, so
    each output must be the round-to-nearest-even bf16 of the exact value, bit
    for bit."""
    c = WL.onebit_case(2048, 4096, 14336, "bf16", "f16", "bf16", kind="int_exact", seed=4)
    G.say(c.name)
    Y = G.run_onebit(c)
    ref = WL.round_to(O.onebit_linear(c.X, c.W_sign, c.a, c.b), "bf16")
    bad = Y != ref
    assert not bad.any(), f"{int(bad.sum())} outputs differ; first at {np.argwhere(bad)[0]}"


def test_workload4_prefill_sampled():
    """Quick check of the same launch on a sample of outputs (rows and columns at
    the tile edges included)."""
    c = WL.workload(4)
    G.say(c.name)
    Y = G.run_onebit(c)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(c.M, 48, replace=False))
    cols = np.sort(rng.choice(c.N, 160, replace=False))
    rows = np.unique(np.concatenate([rows, [0, c.M - 1]]))
    cols = np.unique(np.concatenate([cols, [0, 223, 224, c.N - 1]]))
    Yr = O.onebit_linear(c.X[rows], c.W_sign[cols], c.a[cols], c.b)
    S = O.onebit_error_scale(c.X[rows], c.a[cols], c.b)
    r = O.max_normalised_error(Y[np.ix_(rows, cols)], Yr, S)
    G.say(f"  sampled max normalised error {r:.3e}")
    assert r <= G.TOL_GEMM
    assert np.isfinite(Y).all()


@pytest.mark.parametrize("impl", ["auto", "w7"])
def test_prefill_down_projection_sampled(impl, forcer):
    """2048 x 11008 -> 4096 (a Llama-2-7B MLP down projection): the tile-width
    choice takes 256 columns here (auto); w7 checks the 448-column tile with a
    partial last column tile.  Sampled outputs against the oracle."""
    if impl != "auto":
        forcer(gemm=impl)
    c = WL.onebit_case(2048, 11008, 4096, "bf16", "f16", "bf16", seed=21)
    G.say(f"{c.name} [{impl}]")
    Y = G.run_onebit(c, "gemm")
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.choice(c.M, 32, replace=False), [0, c.M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(c.N, 96, replace=False), [0, 255, 256, 447, 448, c.N - 1]]))
    Yr = O.onebit_linear(c.X[rows], c.W_sign[cols], c.a[cols], c.b)
    r = O.max_normalised_error(Y[np.ix_(rows, cols)], Yr, O.onebit_error_scale(c.X[rows], c.a[cols], c.b))
    G.say(f"  sampled max normalised error {r:.3e}")
    assert r <= G.TOL_GEMM and np.isfinite(Y).all()


def test_workload5_dbf():
    c = WL.workload(5)
    G.say(c.name)
    X = G.dev(c.X, "bf16")
    S2p = B.pack_signs(G.signs_dev(c.S2))
    S1p = B.pack_signs(G.signs_dev(c.S1))
    b, m, a = (G.dev(v, "f16") for v in (c.b, c.m, c.a))
    Y, T1 = B.dbf_linear(X, S2p, S1p, b, m, a)
    Y, T1 = G.host64(Y), G.host64(T1)
    # stage 1 against the oracle at the OneBit scale of stage 1
    T1_ref = O.dbf_stage1(c.X, c.S2, c.b, c.m)
    r1 = O.max_normalised_error(T1, T1_ref, O.onebit_error_scale(c.X, c.m, c.b))
    # stage 2 against the oracle applied to the device's T1
    Y2_ref = O.onebit_linear(T1, c.S1, c.a, np.ones(c.Kmid))
    r2 = O.max_normalised_error(Y, Y2_ref, O.onebit_error_scale(T1, c.a, np.ones(c.Kmid)))
    # composed
    Y_ref = O.dbf_linear(c.X, c.S1, c.S2, c.a, c.m, c.b)
    r = O.max_normalised_error(Y, Y_ref, O.dbf_error_scale(c.X, c.b, c.m, c.a))
    G.say(f"  stage1 {r1:.3e} stage2 {r2:.3e} composed {r:.3e}")
    assert r1 <= G.TOL_DECODE and r2 <= G.TOL_DECODE and r <= G.TOL_DECODE


@pytest.mark.parametrize("path,M,x_dtype,decode", [("lut", 1, "bf16", None), ("lut", 2, "bf16", None),
                                                   ("decode", 4, "bf16", None), ("decode", 16, "bf16", None),
                                                   ("decode", 16, "bf16", "split"), ("decode", 8, "f32", None),
                                                   ("decode", 24, "bf16", None)])
def test_k32768_decode_tolerance(path, M, x_dtype, decode, forcer):
    """K = 32768 on every decode kernel (8 LUT slabs, 8 slices per whole-K wave,
    64 split slices): the slab and slice sums are combined with compensated
    summation, so the 1e-5 bound holds at long K too."""
    if decode:
        forcer(decode=decode)
    K, N = 32768, 160
    G.say(f"K=32768 {path} M={M} x={x_dtype} decode={decode}")
    c = WL.onebit_case(M, K, N, x_dtype, "f16", "f32", seed=M + 33)
    r = G.check_onebit(c, G.run_onebit(c, path), path)
    G.say(f"  max normalised error {r:.3e}")


@pytest.mark.parametrize("path,M", [("lut", 1), ("lut", 2), ("decode", 16), ("gemm", 64), ("gemm", 300)])
def test_long_k(path, M):
    """K = 20480: several GEMV slabs, 40 decode slices, and for the GEMM a K
    whose bf16(b) table no longer fits next to the main kernel's stage
    buffers (the prefill path falls back to the LDS-staged kernel)."""
    K, N = 20480, 300
    G.say(f"long K {path} M={M} K={K} N={N}")
    c = WL.onebit_case(M, K, N, seed=M + 7)
    G.check_onebit(c, G.run_onebit(c, path), path)


# ------------------------------------------------------------------ exact regimes
@pytest.mark.parametrize("path,M,K,N", [("lut", 1, 4096, 1000), ("lut", 2, 8224, 77),
                                        ("decode", 16, 4096, 4096), ("decode", 9, 544, 65),
                                        ("gemm", 300, 4096, 500), ("gemm", 2048, 1024, 448),
                                        ("gemm", 512, 640, 448), ("gemm", 96, 160, 100)])
def test_integer_exact_bitwise(path, M, K, N):
    G.say(f"int-exact {path} M={M} K={K} N={N}")
    c = WL.onebit_case(M, K, N, "bf16", "f16", "f32", kind="int_exact", seed=K + N)
    Y = G.run_onebit(c, path)
    assert np.array_equal(Y, O.onebit_linear(c.X, c.W_sign, c.a, c.b))


@pytest.mark.parametrize("impl", ["w7", "w4", "w2", "w1"])
@pytest.mark.parametrize("M,K,N", [(300, 4096, 500), (129, 640, 449), (130, 128, 500), (70, 256, 257),
                                   (513, 384, 230)])
def test_integer_exact_gemm_tiles(M, K, N, impl, forcer):
    """Every tile of the main prefill kernel, whole K over 1, 2, 3, 5 and 32
    stages (and split K where the grid is small): integer-valued inputs make
    every partial sum exact in fp32, so the result equals the oracle bit for
    bit whatever the order of accumulation."""
    forcer(gemm=impl)
    G.say(f"int-exact gemm[{impl}] M={M} K={K} N={N}")
    c = WL.onebit_case(M, K, N, "bf16", "f16", "f32", kind="int_exact", seed=K + N + M)
    Y = G.run_onebit(c, "gemm")
    assert np.array_equal(Y, O.onebit_linear(c.X, c.W_sign, c.a, c.b))


@pytest.mark.parametrize("path", ["gemm"])
def test_integer_exact_bf16_output_is_rne_of_exact(path):
    c = WL.onebit_case(64, 1024, 224, "bf16", "f16", "bf16", kind="int_exact", seed=3)
    Y = G.run_onebit(c, path)
    assert np.array_equal(Y, WL.round_to(O.onebit_linear(c.X, c.W_sign, c.a, c.b), "bf16"))


@pytest.mark.parametrize("K", [512, 4096])
@pytest.mark.parametrize("path,M", [("lut", 1), ("lut", 2), ("decode", 16), ("gemm", None)])
def test_hadamard_closed_form(K, path, M):
    """Sylvester Hadamard: X = H[:M], W_sign = H, a = b = 1 gives K·I[:M] exactly."""
    G.say(f"hadamard K={K} {path}")
    H = WL.sylvester_hadamard(K)
    M = M or K
    X = G.dev(H[:M].astype(np.float64), "bf16")
    Wp = B.pack_signs(G.signs_dev(H))
    one = torch.ones(K, dtype=torch.float16, device="cuda")
    with G.forced_path(path):
        Y = G.host64(B.linear(X, Wp, one, one))
    assert np.array_equal(Y, K * np.eye(K)[:M])


@pytest.mark.parametrize("path,M", [("lut", 2), ("decode", 16), ("gemm", 64)])
def test_random_x_against_fwht(path, M):
    K = 1024
    H = WL.sylvester_hadamard(K)
    rng = np.random.default_rng(M)
    Xv = WL.round_to(rng.standard_normal((M, K)), "bf16")
    one = torch.ones(K, dtype=torch.float16, device="cuda")
    with G.forced_path(path):
        Y = G.host64(B.linear(G.dev(Xv, "bf16"), B.pack_signs(G.signs_dev(H)), one, one))
    S = np.abs(Xv).sum(axis=1, keepdims=True) * np.ones((1, K))
    tol = G.TOL_GEMM if path == "gemm" else G.TOL_DECODE
    assert O.max_normalised_error(Y, fwht_rows(Xv), S) <= tol


@pytest.mark.parametrize("path", ["lut", "decode", "gemm"])
def test_page_example_padded(path):
    """LLM.int8() page, section 4.2.1: hidden @ pm1 then softmax = [0, .5, .5, 0].
    K = 4 is zero-padded to 32 (X) and +1-padded (signs)."""
    g = json.load(open(os.path.join(GOLDEN, "llm_int8_emergent_pm1_example.json")))
    Hd = np.array(g["hidden"], dtype=np.float64)
    Pm = np.array(g["pm1_matrix"], dtype=np.int8)
    X = np.zeros((4, 32))
    X[:, :4] = Hd
    S = np.ones((4, 32), dtype=np.int8)
    S[:, :4] = Pm.T
    one = torch.ones(32, dtype=torch.float32, device="cuda")
    Wp = B.pack_signs(G.signs_dev(S))
    rows = [X[0:1], X[1:2], X[2:3], X[3:4]] if path == "lut" else [X]
    outs = []
    with G.forced_path(path):
        for xr in rows:
            outs.append(G.host64(B.linear(G.dev(xr, "f32"), Wp, one[:4], one)))
    Y = np.vstack(outs)
    assert np.array_equal(Y, Hd @ Pm.astype(np.float64))
    e = np.exp(Y - Y.max(axis=1, keepdims=True))
    sm = np.round(e / e.sum(axis=1, keepdims=True), g["printed_decimals"])
    assert np.array_equal(sm, np.array(g["softmax_of_product"], dtype=np.float64))


# ------------------------------------------------------------------ DBF
@pytest.mark.parametrize("path,M", [("lut", 1), ("lut", 2), ("decode", 8), ("decode", 16)])
def test_dbf_integer_exact(path, M):
    G.say(f"dbf int-exact {path} M={M}")
    c = WL.dbf_case(M, 4096, 3072, 4096, kind="int_exact", seed=M)
    X = G.dev(c.X, "bf16")
    S2p = B.pack_signs(G.signs_dev(c.S2))
    S1p = B.pack_signs(G.signs_dev(c.S1))
    b, m, a = (G.dev(v, "f16") for v in (c.b, c.m, c.a))
    with G.forced_path(path):
        Y, T1 = B.dbf_linear(X, S2p, S1p, b, m, a)
    assert np.array_equal(G.host64(T1), O.dbf_stage1(c.X, c.S2, c.b, c.m))
    assert np.array_equal(G.host64(Y), O.dbf_linear(c.X, c.S1, c.S2, c.a, c.m, c.b))


@pytest.mark.parametrize("path,M,K,Kmid,N", [("lut", 1, 512, 96, 130), ("decode", 5, 544, 160, 100),
                                             ("decode", 16, 1024, 512, 1024)])
def test_dbf_parity_and_two_calls(path, M, K, Kmid, N):
    G.say(f"dbf {path} M={M} K={K} Kmid={Kmid} N={N}")
    c = WL.dbf_case(M, K, Kmid, N, seed=K + N)
    X = G.dev(c.X, "bf16")
    S2p = B.pack_signs(G.signs_dev(c.S2))
    S1p = B.pack_signs(G.signs_dev(c.S1))
    b, m, a = (G.dev(v, "f16") for v in (c.b, c.m, c.a))
    with G.forced_path(path):
        Y, T1 = B.dbf_linear(X, S2p, S1p, b, m, a)
        T1b = B.linear(X, S2p, m, b)
        Yb = B.linear(T1b, S1p, a, torch.ones(Kmid, dtype=torch.float16, device="cuda"))
    Yh = G.host64(Y)
    assert torch.equal(T1, T1b) and torch.equal(Y, Yb)
    r = O.max_normalised_error(Yh, O.dbf_linear(c.X, c.S1, c.S2, c.a, c.m, c.b),
                               O.dbf_error_scale(c.X, c.b, c.m, c.a))
    assert r <= G.TOL_DECODE


@pytest.mark.parametrize("M", [32, 300])
def test_dbf_prefill(M):
    G.say(f"dbf prefill M={M}")
    c = WL.dbf_case(M, 1024, 512, 448, seed=M)
    X = G.dev(c.X, "bf16")
    S2p = B.pack_signs(G.signs_dev(c.S2))
    S1p = B.pack_signs(G.signs_dev(c.S1))
    b, m, a = (G.dev(v, "f16") for v in (c.b, c.m, c.a))
    Y, T1 = B.dbf_linear(X, S2p, S1p, b, m, a, out_dtype=torch.bfloat16)
    r1 = O.max_normalised_error(G.host64(T1), O.dbf_stage1(c.X, c.S2, c.b, c.m),
                                O.onebit_error_scale(c.X, c.m, c.b))
    r = O.max_normalised_error(G.host64(Y), O.dbf_linear(c.X, c.S1, c.S2, c.a, c.m, c.b),
                               O.dbf_error_scale(c.X, c.b, c.m, c.a))
    G.say(f"  stage1 {r1:.3e} composed {r:.3e}")
    assert r1 <= G.TOL_GEMM and r <= G.TOL_DBF_GEMM


@pytest.mark.parametrize("Kmid", [2048, 3072, 4736])
def test_dbf_prefill_full_size(Kmid):
    """DBF prefill at M = 512 with K = N = 4096 and Kmid for 1.0 / 1.5 / 2.3 sign
    bits per weight (DBF page, "Belangrijkste Bijdragen": the middle dimension
    sets the ratio).  Sampled rows against the oracle, stage 1 and composed."""
    M = 512
    G.say(f"dbf prefill M={M} Kmid={Kmid}")
    c = WL.dbf_case(M, 4096, Kmid, 4096, seed=Kmid)
    X = G.dev(c.X, "bf16")
    S2p = B.pack_signs(G.signs_dev(c.S2))
    S1p = B.pack_signs(G.signs_dev(c.S1))
    b, m, a = (G.dev(v, "f16") for v in (c.b, c.m, c.a))
    Y, T1 = B.dbf_linear(X, S2p, S1p, b, m, a, out_dtype=torch.bfloat16)
    rows = np.unique(np.concatenate([np.random.default_rng(Kmid).choice(M, 20, replace=False), [0, M - 1]]))
    r1 = O.max_normalised_error(G.host64(T1)[rows], O.dbf_stage1(c.X[rows], c.S2, c.b, c.m),
                                O.onebit_error_scale(c.X[rows], c.m, c.b))
    r = O.max_normalised_error(G.host64(Y)[rows], O.dbf_linear(c.X[rows], c.S1, c.S2, c.a, c.m, c.b),
                               O.dbf_error_scale(c.X[rows], c.b, c.m, c.a))
    G.say(f"  stage1 {r1:.3e} composed {r:.3e}")
    assert r1 <= G.TOL_GEMM and r <= G.TOL_DBF_GEMM


# ------------------------------------------------------------------ determinism, edge cases
@pytest.mark.parametrize("path,M", [("lut", 1), ("decode", 16), ("gemm", 256)])
def test_bitwise_reproducible(path, M):
    c = WL.onebit_case(M, 4096, 4096, seed=M)
    X = G.dev(c.X, "bf16")
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    a, b = G.dev(c.a, "f16"), G.dev(c.b, "f16")
    with G.forced_path(path):
        ref = B.linear(X, Wp, a, b)
        for _ in range(20):
            assert torch.equal(B.linear(X, Wp, a, b), ref)


def test_m0_returns_empty():
    Wp = B.pack_signs(torch.ones((8, 32), dtype=torch.int8, device="cuda"))
    X = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    one = torch.ones(32, dtype=torch.float16, device="cuda")
    Y = B.linear(X, Wp, one[:8], one)
    assert Y.shape == (0, 8)


def test_alias_rejected_on_device():
    X = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    Wp = B.pack_signs(torch.ones((4, 64), dtype=torch.int8, device="cuda"))
    one = torch.ones(64, dtype=torch.float32, device="cuda")
    with pytest.raises(B.OblError) as e:
        B.linear(X, Wp, one[:4], one, out=X.view(-1)[:16].view(4, 4))
    assert e.value.status == B.OBL_ERR_ALIAS


def test_streams_are_respected():
    """Work enqueued on a side stream is ordered with that stream's events."""
    c = WL.onebit_case(1, 4096, 2048, seed=8)
    X = G.dev(c.X, "bf16")
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    a, b = G.dev(c.a, "f16"), G.dev(c.b, "f16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Y = B.linear(X, Wp, a, b)
    s.synchronize()
    G.check_onebit(c, G.host64(Y))
