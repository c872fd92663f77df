"""Library scratch on the GPU: per-stream pools, growth refused inside stream
capture (and the capture left valid), graphs that keep working after the pool
grows, concurrent streams, and kernel choice independent of the environment.

The calls used need scratch: fp32 activations at decode sizes run the split
kernel, whose per-slice partial sums live in the pool of the call's stream.
"""
import os

import numpy as np
import pytest
import torch

from tests import gpu_util as G
import oracle as O
from bit_weight_linear_amd import binding as B
from bit_weight_linear_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _split_case(M, K, N, seed):
    c = WL.onebit_case(M, K, N, "f32", "f32", "f32", seed=seed)
    return c, G.dev(c.X, "f32"), B.pack_signs(G.signs_dev(c.W_sign)), G.dev(c.a, "f32"), G.dev(c.b, "f32")


def test_growth_inside_capture_is_refused_and_capture_stays_valid():
    """A fresh stream has an empty pool: the first scratch-using call inside a
    capture returns OBL_ERR_CAPTURE and enqueues nothing; the capture still
    ends normally, and after one eager call on that stream the same call can
    be captured and replayed."""
    c, X, Wp, a, b = _split_case(4, 4096, 512, seed=1)
    B.linear(X, Wp, a, b)                # eager on the current stream: device queries done outside capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    Y = torch.zeros((4, 512), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(g, stream=s):
        try:
            B.linear(X, Wp, a, b, out=Y)
        except B.OblError as e:
            status = e.status
        Y.add_(1.0)                      # the capture goes on after the refusal
    assert status == B.OBL_ERR_CAPTURE
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(Y, torch.ones_like(Y))
    # Sized by one eager call on the stream, the call captures and replays.
    with torch.cuda.stream(s):
        B.linear(X, Wp, a, b, out=Y)
    s.synchronize()
    ref = Y.clone()
    Y.zero_()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s):
        B.linear(X, Wp, a, b, out=Y)
    for _ in range(3):
        Y.zero_()
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref)
    G.check_onebit(c, G.host64(Y))


def test_graph_replays_after_the_pool_grows():
    """Capture a scratch-using call, then make the pool grow with a larger eager
    call on the same stream, then replay: the captured call still uses its
    (retired but never freed) buffer and gives the same result every time."""
    c, X, Wp, a, b = _split_case(2, 2048, 256, seed=2)
    s = torch.cuda.Stream()
    Y = torch.empty((2, 256), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        B.linear(X, Wp, a, b, out=Y)          # sizes the pool of s for this call
    s.synchronize()
    ref = Y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.linear(X, Wp, a, b, out=Y)
    # A call that needs far more than the pool holds: 16 x 16384 x 8192 in fp32
    # takes 32 slices x 16 x 8192 floats = 16 MiB of partial sums.
    cb, Xb, Wb, ab, bb = _split_case(16, 16384, 8192, seed=3)
    Yb = torch.empty((16, 8192), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        B.linear(Xb, Wb, ab, bb, out=Yb)
    s.synchronize()
    G.check_onebit(cb, G.host64(Yb))
    for _ in range(3):
        Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref)


def test_two_streams_concurrently():
    """The split decode kernel on two streams at once (each with its own pool):
    both results equal the eager ones computed one at a time."""
    cases = [_split_case(8, 8192, 4096, seed=10 + i) for i in range(2)]
    refs = []
    for c, X, Wp, a, b in cases:
        refs.append(B.linear(X, Wp, a, b))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(r) for r in refs]
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for (c, X, Wp, a, b), s, o in zip(cases, streams, outs):
            with torch.cuda.stream(s):
                for _ in range(3):
                    B.linear(X, Wp, a, b, out=o)
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r)
    for (c, *_), o in zip(cases, outs):
        G.check_onebit(c, G.host64(o))


def test_environment_does_not_choose_the_kernel():
    """The library reads no environment variable: with OBL_PATH=gemm (the name a
    test switch once had) an M = 1 call still takes the decode GEMV and meets
    the 1e-5 bound."""
    c = WL.onebit_case(1, 4096, 1000, seed=5)
    old = os.environ.get("OBL_PATH")
    os.environ["OBL_PATH"] = "gemm"
    os.environ["OBL_GEMM"] = "v1"
    try:
        Y = G.run_onebit(c)
    finally:
        os.environ.pop("OBL_GEMM", None)
        if old is None:
            os.environ.pop("OBL_PATH", None)
        else:
            os.environ["OBL_PATH"] = old
    r = G.check_onebit(c, Y)
    assert r <= G.TOL_DECODE
