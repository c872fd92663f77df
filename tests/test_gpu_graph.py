"""The library's calls inside a captured HIP graph: every replay must equal the
eager result bitwise (the kernels are deterministic and use no memset nodes).
Replays are interleaved with unrelated eager work and synchronisations."""
import numpy as np
import pytest
import torch

from bit_weight_linear_amd import workloads as WL
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

B = pytest.importorskip("bit_weight_linear_amd.binding", reason="libobl.so not built")


def _replays_match(fn, outs):
    """fn() writes into the tensors `outs`; capture it, replay 3 times, compare."""
    fn()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                              # warm-up on the capture stream: sizes that stream's library scratch
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda")
        (junk * 2).sum().item()           # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from the eager result"


@pytest.mark.parametrize("M", [1, 2, 8, 16, 64, 512])
def test_linear_in_graph(M):
    G.say(f"graph linear M={M}")
    c = WL.onebit_case(M, 4096, 1024, seed=M)
    X, a, b = G.dev(c.X, "bf16"), G.dev(c.a, "f16"), G.dev(c.b, "f16")
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    Y = torch.empty((M, 1024), dtype=torch.float32, device="cuda")
    _replays_match(lambda: B.linear(X, Wp, a, b, out=Y), [Y])


def test_linear_fp32_activations_prefill_in_graph():
    c = WL.onebit_case(96, 2048, 448, x_dtype="f32", seed=5)
    X, a, b = G.dev(c.X, "f32"), G.dev(c.a, "f16"), G.dev(c.b, "f16")
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    Y = torch.empty((96, 448), dtype=torch.float32, device="cuda")
    _replays_match(lambda: B.linear(X, Wp, a, b, out=Y), [Y])


@pytest.mark.parametrize("M", [4, 512])
def test_dbf_in_graph(M):
    c = WL.dbf_case(M, 4096, 3072, 4096, seed=M)
    X = G.dev(c.X, "bf16")
    S2p, S1p = B.pack_signs(G.signs_dev(c.S2)), B.pack_signs(G.signs_dev(c.S1))
    b, m, a = (G.dev(v, "f16") for v in (c.b, c.m, c.a))
    Y = torch.empty((M, 4096), dtype=torch.float32, device="cuda")
    ws = torch.empty((M, 3072), dtype=torch.float32, device="cuda")
    _replays_match(lambda: B.dbf_linear(X, S2p, S1p, b, m, a, workspace=ws, out=Y), [Y, ws])


def test_backward_and_layernorm_in_graph():
    M, K, N = 16, 1024, 512
    c = WL.onebit_case(M, K, N, seed=3)
    rng = np.random.default_rng(4)
    dY = G.dev(WL.round_to(rng.standard_normal((M, N)), "bf16"), "bf16")
    X, a, b = G.dev(c.X, "bf16"), G.dev(c.a, "f16"), G.dev(c.b, "f16")
    Wp = B.pack_signs(G.signs_dev(c.W_sign))
    Wt = B.transpose_signs(Wp, N, K)
    ws = torch.empty(M * (N + K), dtype=torch.float32, device="cuda")
    outs = {}

    def bwd():
        dX, da, db, _ = B.linear_backward(dY, X, Wp, Wt, a, b, workspace=ws)
        outs["r"] = (dX, da, db)
    # the binding allocates dX, da, db per call: capture writes into graph-owned
    # tensors, so compare through fixed copies
    dX0 = torch.empty((M, K), device="cuda")
    da0, db0 = torch.empty(N, device="cuda"), torch.empty(K, device="cuda")

    def bwd_into():
        bwd()
        dX0.copy_(outs["r"][0]); da0.copy_(outs["r"][1]); db0.copy_(outs["r"][2])
    _replays_match(bwd_into, [dX0, da0, db0])

    Z = torch.empty((M, N), dtype=torch.float32, device="cuda")
    wsl = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _replays_match(lambda: B.linear_layernorm(X, Wp, a, b, 1e-5, workspace=wsl, out=Z), [Z, wsl])
