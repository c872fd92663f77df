"""Decode path (3 <= M <= 32): the whole-K kernel against the fp64 oracle, and
against the split-K kernel (M <= 16).

The whole-K kernel serves bf16 x with fp16 b, 16-byte aligned X and packed
words, K % 128 == 0: one workgroup of 8 waves owns 16·CPW columns over all of
K (CPW = 1, 2 or 4 column groups per wave), wave w contracts the 512-k slices
w, w + 8, ..., and the waves' sums are added in wave order.  OBL_DECODE forces
the kernel (split, wk1, wk2, wk4).  Tolerance: the decode path's 1e-5 on the
normalised scale (fp32 contraction with exact products).
"""
import numpy as np
import pytest
import torch

from tests import gpu_util as G
import oracle as O
from bit_weight_linear_amd import binding as B
from bit_weight_linear_amd import workloads as WL

pytestmark = pytest.mark.gpu

# (M, K, N): one partial slice (K = 128); two slices, the second of 4 steps
# (K = 640); N not a multiple of the column block; two and five slices per
# wave (K = 8192, 20480); the batched-decode shape and its 14336-wide variant.
# 17..32 rows (two 16-row fragments, 4 waves per workgroup): ragged fragment
# (17, 20), two slices per wave at K = 4096, a partial last slice (K = 640).
WK_CASES = [
    (3, 128, 17), (5, 640, 100), (9, 4096, 1000), (16, 8192, 129), (16, 20480, 300),
    (16, 4096, 4096), (16, 4096, 14336), (8, 4096, 3072), (16, 1024, 65),
    (17, 4096, 1000), (20, 640, 100), (24, 8192, 129), (32, 4096, 4096), (32, 4096, 14336),
]
IMPLS = ["wk1", "wk2", "wk4", "split", "auto"]


@pytest.mark.parametrize("M,K,N", WK_CASES)
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
@pytest.mark.parametrize("impl", IMPLS)
def test_decode_kernels_match_oracle(M, K, N, ydt, impl, forcer):
    G.say(f"decode {impl} M={M} K={K} N={N} y={ydt}")
    forcer(decode=impl)
    c = WL.onebit_case(M, K, N, "bf16", "f16", ydt, seed=M * 7 + K + N)
    if impl == "split" and M > 16:
        # the split kernel stages 16 rows: a forced decode call is refused
        with pytest.raises(B.OblError) as e:
            G.run_onebit(c, "decode")
        assert e.value.status == B.OBL_ERR_SHAPE
        return
    r = G.check_onebit(c, G.run_onebit(c, "decode"), "decode")
    G.say(f"  max normalised error {r:.3e}")


@pytest.mark.parametrize("M", [17, 24, 32])
def test_mid_rows_default_to_whole_k(M):
    """17..32 rows with bf16 x, fp16 scales and aligned operands take the
    whole-K decode kernel by default: the decode path's 1e-5 bound holds."""
    c = WL.onebit_case(M, 4096, 1000, "bf16", "f16", "f32", seed=M)
    G.check_onebit(c, G.run_onebit(c), "decode")


def test_mid_rows_fp32_x_take_the_gemm():
    """fp32 x at 24 rows is not a whole-K call: the prefill GEMM serves it
    (its 8e-3 bound), and a forced decode call is refused."""
    c = WL.onebit_case(24, 1024, 300, "f32", "f32", "f32", seed=4)
    G.check_onebit(c, G.run_onebit(c), "gemm")
    with pytest.raises(B.OblError) as e:
        G.run_onebit(c, "decode")
    assert e.value.status == B.OBL_ERR_SHAPE


@pytest.mark.parametrize("M,K,N", [(16, 4096, 4096), (7, 2048, 1000), (16, 640, 33)])
def test_whole_k_one_group_is_bitwise_the_split_kernel(M, K, N, forcer):
    """K <= 4096 with one column group per wave adds the same fp32 terms in the
    same order as the split kernel and its slice reduction."""
    c = WL.onebit_case(M, K, N, "bf16", "f16", "f32", seed=K + N)
    X = G.dev(c.X, "bf16")
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    a, b = G.dev(c.a, "f16"), G.dev(c.b, "f16")
    out = {}
    for impl in ("wk1", "split"):
        forcer(decode=impl)
        with G.forced_path("decode"):
            out[impl] = B.linear(X, Wp, a, b)
    torch.cuda.synchronize()
    assert torch.equal(out["wk1"], out["split"])


@pytest.mark.parametrize("impl", ["wk1", "wk2", "wk4"])
def test_whole_k_integer_exact_and_reproducible(impl, forcer):
    """Integer-valued inputs: every partial sum is exact in fp32, so the result
    equals the oracle exactly; repeated calls are bitwise equal."""
    forcer(decode=impl)
    c = WL.onebit_case(16, 4096, 1000, "bf16", "f16", "f32", kind="int_exact", seed=3)
    X = G.dev(c.X, "bf16")
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    a, b = G.dev(c.a, "f16"), G.dev(c.b, "f16")
    with G.forced_path("decode"):
        ref = B.linear(X, Wp, a, b)
        for _ in range(5):
            assert torch.equal(B.linear(X, Wp, a, b), ref)
    assert np.array_equal(G.host64(ref), O.onebit_linear(c.X, c.W_sign, c.a, c.b))


def test_whole_k_offset_operands_use_split_kernel(forcer):
    """X 2 bytes past a 16-byte boundary is not DMA-able: the call must still
    be right (the split kernel's element staging takes it)."""
    forcer(decode="wk1")
    M, K, N = 4, 1024, 200
    c = WL.onebit_case(M, K, N, "bf16", "f16", "f32", seed=5)
    big = torch.zeros(M * K + 1, dtype=torch.bfloat16, device="cuda")
    X = big[1:].view(M, K)
    X.copy_(G.dev(c.X, "bf16"))
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    with G.forced_path("decode"):
        Y = B.linear(X, Wp, G.dev(c.a, "f16"), G.dev(c.b, "f16"))
    G.check_onebit(c, G.host64(Y), "decode")


@pytest.mark.parametrize("impl", ["wk1", "split"])
def test_dbf_decode_stage1_whole_k(impl, forcer):
    """DBF decode: stage 1 (bf16 x, fp16 b) runs on the kernel under test,
    stage 2 (fp32 T1) on the split kernel."""
    forcer(decode=impl)
    c = WL.workload(5)
    X = G.dev(c.X, "bf16")
    S2p = B.pack_signs(G.signs_dev(c.S2))
    S1p = B.pack_signs(G.signs_dev(c.S1))
    b, m, a = (G.dev(v, "f16") for v in (c.b, c.m, c.a))
    Y, T1 = B.dbf_linear(X, S2p, S1p, b, m, a)
    r1 = O.max_normalised_error(G.host64(T1), O.dbf_stage1(c.X, c.S2, c.b, c.m),
                                O.onebit_error_scale(c.X, c.m, c.b))
    r = O.max_normalised_error(G.host64(Y), O.dbf_linear(c.X, c.S1, c.S2, c.a, c.m, c.b),
                               O.dbf_error_scale(c.X, c.b, c.m, c.a))
    G.say(f"dbf {impl}: stage1 {r1:.3e} composed {r:.3e}")
    assert r1 <= G.TOL_DECODE and r <= G.TOL_DECODE


@pytest.mark.parametrize("impl", ["auto", "wk1", "wk2", "wk4"])
@pytest.mark.parametrize("M,K,Kmid,N", [(8, 4096, 3072, 4096), (3, 1024, 640, 300), (5, 4096, 4096, 1000),
                                        (8, 512, 128, 4096)])
def test_dbf_decode_through_exact_terms(M, K, Kmid, N, impl, forcer):
    """Up to 8 rows with both stages on the whole-K kernel: stage 1 writes the
    exact bf16 terms (hi + mid + lo) of T1 and stage 2 contracts them against
    the signs of S1.  T1 is bitwise the single-stage result; both stages meet
    the decode tolerance against the oracle."""
    if impl != "auto":
        forcer(decode=impl)
    G.say(f"dbf terms {impl} M={M} K={K} Kmid={Kmid} N={N}")
    c = WL.dbf_case(M, K, Kmid, N, seed=K + Kmid + N + M)
    X = G.dev(c.X, "bf16")
    S2p = B.pack_signs(G.signs_dev(c.S2))
    S1p = B.pack_signs(G.signs_dev(c.S1))
    b, m, a = (G.dev(v, "f16") for v in (c.b, c.m, c.a))
    Y, T1 = B.dbf_linear(X, S2p, S1p, b, m, a)
    T1b = B.linear(X, S2p, m, b)
    assert torch.equal(T1, T1b)
    Th = G.host64(T1)
    r1 = O.max_normalised_error(Th, O.dbf_stage1(c.X, c.S2, c.b, c.m), O.onebit_error_scale(c.X, c.m, c.b))
    # stage 2 against the oracle applied to the device's T1 (the terms carry T1 exactly)
    r2 = O.max_normalised_error(G.host64(Y), O.onebit_linear(Th, c.S1, c.a, np.ones(Kmid)),
                                O.onebit_error_scale(Th, c.a, np.ones(Kmid)))
    r = O.max_normalised_error(G.host64(Y), O.dbf_linear(c.X, c.S1, c.S2, c.a, c.m, c.b),
                               O.dbf_error_scale(c.X, c.b, c.m, c.a))
    G.say(f"  stage1 {r1:.3e} stage2 {r2:.3e} composed {r:.3e}")
    assert r1 <= G.TOL_DECODE and r2 <= G.TOL_DECODE and r <= G.TOL_DECODE


def test_dbf_decode_terms_integer_exact():
    """Integer-valued DBF at 8 rows through the exact terms: bit-exact."""
    c = WL.dbf_case(8, 4096, 3072, 4096, kind="int_exact", seed=8)
    X = G.dev(c.X, "bf16")
    S2p = B.pack_signs(G.signs_dev(c.S2))
    S1p = B.pack_signs(G.signs_dev(c.S1))
    b, m, a = (G.dev(v, "f16") for v in (c.b, c.m, c.a))
    Y, T1 = B.dbf_linear(X, S2p, S1p, b, m, a)
    assert np.array_equal(G.host64(T1), O.dbf_stage1(c.X, c.S2, c.b, c.m))
    assert np.array_equal(G.host64(Y), O.dbf_linear(c.X, c.S1, c.S2, c.a, c.m, c.b))
