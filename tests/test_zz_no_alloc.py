"""dbf_linear_noalloc: the allocation-free variant of dbf_linear, whose library
scratch is a fixed device array.  Checked against dbf_linear on the same inputs
-- bitwise, since both run the same kernels in the same order -- on two calls
in a row, the second with a smaller input, at decode and prefill sizes; and a
call that needs more scratch than the array holds is refused before any work.
"""
import numpy as np
import pytest
import torch

from tests import gpu_util as G
import oracle as O
from bit_weight_linear_amd import binding as B
from bit_weight_linear_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _dev_case(c):
    X = G.dev(c.X, c.x_dtype)
    S2 = B.pack_signs(G.signs_dev(c.S2))
    S1 = B.pack_signs(G.signs_dev(c.S1))
    sc = [G.dev(v, c.scale_dtype) for v in (c.b, c.m, c.a)]
    return X, S2, S1, sc


def _both(c, y_dtype):
    X, S2, S1, sc = _dev_case(c)
    M, Kmid, N = c.X.shape[0], c.S2.shape[0], c.S1.shape[0]
    Y0, T0 = B.dbf_linear(X, S2, S1, *sc, out_dtype=y_dtype)
    ws = torch.full((M, Kmid), float("nan"), dtype=torch.float32, device="cuda")
    Y1 = torch.full((M, N), float("nan"), dtype=y_dtype, device="cuda")
    B.dbf_linear_noalloc(X, S2, S1, *sc, workspace=ws, out=Y1)
    torch.cuda.synchronize()
    return (Y0, T0), (Y1, ws)


@pytest.mark.parametrize("shapes,y_dtype,tol", [
    # decode: stage 1 writes the exact bf16 terms of T1 into the fixed array
    (((8, 4096, 3072, 4096), (4, 1024, 512, 768)), torch.float32, G.TOL_DECODE),
    # prefill: the bf16 copy of T1 in slot 0; the second call splits K (slot 1)
    (((512, 4096, 3072, 4096), (64, 1024, 640, 512)), torch.bfloat16, G.TOL_DBF_GEMM),
])
def test_noalloc_matches_dbf_linear_twice(shapes, y_dtype, tol):
    for i, (M, K, Kmid, N) in enumerate(shapes):
        G.say(f"noalloc call {i}: M={M} K={K} Kmid={Kmid} N={N}")
        c = WL.dbf_case(M, K, Kmid, N, seed=17 + i)
        (Y0, T0), (Y1, T1) = _both(c, y_dtype)
        assert torch.equal(Y1, Y0), "output differs from dbf_linear"
        assert torch.equal(T1, T0), "workspace (T1) differs from dbf_linear"
        r = O.max_normalised_error(G.host64(Y1), O.dbf_linear(c.X, c.S1, c.S2, c.a, c.m, c.b),
                                   O.dbf_error_scale(c.X, c.b, c.m, c.a))
        G.say(f"  max normalised error {r:.3e}")
        assert r <= tol


def test_noalloc_refuses_more_than_the_array():
    """M Kmid bf16 values of T1 beyond the 32 MiB slot: OBL_ERR_SCRATCH, and the
    output is untouched (nothing was enqueued)."""
    M, K, Kmid, N = 4096, 128, 8192, 128
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    S2 = torch.zeros((Kmid, K // 32), dtype=torch.int32, device="cuda")
    S1 = torch.zeros((N, Kmid // 32), dtype=torch.int32, device="cuda")
    b = torch.ones(K, dtype=torch.float16, device="cuda")
    m = torch.ones(Kmid, dtype=torch.float16, device="cuda")
    a = torch.ones(N, dtype=torch.float16, device="cuda")
    ws = torch.empty((M, Kmid), dtype=torch.float32, device="cuda")
    Y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.OblError) as e:
        B.dbf_linear_noalloc(X, S2, S1, b, m, a, workspace=ws, out=Y)
    assert e.value.status == B.OBL_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())


@pytest.mark.parametrize("M,K,Kmid,N,y_dtype", [(8, 4096, 3072, 4096, torch.float32),
                                                (512, 4096, 3072, 4096, torch.bfloat16)])
def test_noalloc_in_graph_on_a_fresh_stream(M, K, Kmid, N, y_dtype):
    """The allocation-free call captured on a stream the library has never
    seen (so it has no per-stream scratch): every replay, with unrelated eager
    work between replays, equals the eager result bitwise."""
    G.say(f"noalloc graph M={M} K={K} Kmid={Kmid} N={N}")
    c = WL.dbf_case(M, K, Kmid, N, seed=29)
    X, S2, S1, sc = _dev_case(c)
    ws = torch.empty((M, Kmid), dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=y_dtype, device="cuda")
    B.dbf_linear_noalloc(X, S2, S1, *sc, workspace=ws, out=Y)   # eager, on the current stream
    torch.cuda.synchronize()
    ref_y, ref_ws = Y.clone(), ws.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.dbf_linear_noalloc(X, S2, S1, *sc, workspace=ws, out=Y)
    torch.cuda.synchronize()
    for rep in range(3):
        Y.fill_(float("nan"))
        ws.fill_(float("nan"))
        (torch.randn(1 << 20, device="cuda") * 2).sum().item()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref_y), f"replay {rep}: output differs from the eager call"
        assert torch.equal(ws, ref_ws), f"replay {rep}: workspace differs from the eager call"
