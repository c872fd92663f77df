"""CPU tests of the binding's argument checks: every shape, dtype and
scale-dtype mismatch is refused with ValueError before the library is called.

The device check (tensors on the current HIP device) is replaced here by a
contiguity check so the shape checks can run on host tensors; a call that got
past the checks would reach the library, so every case below must raise
first.  Skipped when a GPU is present (host pointers must never reach it).
"""
import pytest
import torch

B = pytest.importorskip("bit_weight_linear_amd.binding", reason="libobl.so not built")

pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="host-tensor checks only run without a GPU")


@pytest.fixture(autouse=True)
def host_tensors(monkeypatch):
    def _dev(t, name):
        if not isinstance(t, torch.Tensor):
            raise TypeError(name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    monkeypatch.setattr(B, "_dev", _dev)

    def no_call(*a, **k):
        raise AssertionError("the library was called")
    monkeypatch.setattr(B, "_check", no_call)


def T(*shape, dt=torch.bfloat16):
    return torch.zeros(shape, dtype=dt)


M, K, N, KM = 4, 256, 96, 128
X, W, a, b = T(M, K), T(N, K // 32, dt=torch.int32), T(N, dt=torch.float16), T(K, dt=torch.float16)


@pytest.mark.parametrize("kw", [
    dict(W_packed=T(N, K // 32 + 1, dt=torch.int32)),     # packed width != K/32
    dict(W_packed=T(N, K // 32, dt=torch.float32)),        # packed dtype
    dict(a=T(N + 1, dt=torch.float16)),                    # a length != N
    dict(b=T(K - 1, dt=torch.float16)),                    # b length != K
    dict(b=T(K, dt=torch.float32)),                        # a f16, b f32
    dict(a=T(N, dt=torch.bfloat16), b=T(K, dt=torch.bfloat16)),   # bf16 scales
    dict(X=T(M, K, dt=torch.float16)),                     # fp16 activations
    dict(X=T(M, K)[:, ::2]),                               # not contiguous
    dict(out=T(M, N + 1, dt=torch.float32)),               # out shape
    dict(out=T(M, N, dt=torch.float16)),                   # out dtype
    dict(X=T(M, 200), W_packed=T(N, 6, dt=torch.int32), b=T(200, dt=torch.float16)),   # K % 32
])
def test_linear_rejects(kw):
    args = dict(X=X, W_packed=W, a=a, b=b)
    args.update(kw)
    with pytest.raises(ValueError):
        B.linear(**args)


S2, S1 = T(KM, K // 32, dt=torch.int32), T(N, KM // 32, dt=torch.int32)
m = T(KM, dt=torch.float16)


@pytest.mark.parametrize("kw", [
    dict(S2_packed=T(KM, K // 32 - 1, dt=torch.int32)),
    dict(S1_packed=T(N, KM // 32 + 1, dt=torch.int32)),
    dict(m=T(KM + 32, dt=torch.float16)),
    dict(m=T(KM, dt=torch.float32)),
    dict(workspace=T(M, KM + 1, dt=torch.float32)),
    dict(workspace=T(M, KM, dt=torch.float16)),
    dict(out=T(M + 1, N, dt=torch.float32)),
])
def test_dbf_rejects(kw):
    args = dict(X=X, S2_packed=S2, S1_packed=S1, b=b, m=m, a=a)
    args.update(kw)
    with pytest.raises(ValueError):
        B.dbf_linear(**args)
    if "workspace" in kw and "out" not in kw:
        args["out"] = T(M, N, dt=torch.float32)
    if "workspace" in args and "out" in args:
        with pytest.raises(ValueError):
            B.dbf_linear_noalloc(**args)


def test_backward_rejects():
    Wt = T(K, N // 32, dt=torch.int32)
    dY = T(M, N)
    with pytest.raises(ValueError):
        B.linear_backward(T(M, N + 1), X, W, Wt, a, b)              # dY shape
    with pytest.raises(ValueError):
        B.linear_backward(T(M, N, dt=torch.float32), X, W, Wt, a, b)   # dY dtype != X dtype
    with pytest.raises(ValueError):
        B.linear_backward(dY, X, W, T(K, N // 32 + 1, dt=torch.int32), a, b)   # transposed packing
    with pytest.raises(ValueError):
        B.linear_backward(dY, X, W, Wt, a, b, workspace=T(M * (N + K) - 1, dt=torch.float32))


def test_layernorm_rejects():
    Y = T(M, N, dt=torch.float32)
    with pytest.raises(ValueError):
        B.layernorm(Y, gamma=T(N + 1, dt=torch.float16))
    with pytest.raises(ValueError):
        B.layernorm(Y, gamma=T(N, dt=torch.float16), beta=T(N, dt=torch.float32))
    with pytest.raises(ValueError):
        B.layernorm(Y, out=T(M, N - 1, dt=torch.float32))
    with pytest.raises(ValueError):
        B.linear_layernorm(X, W, a, b, gamma=T(N, dt=torch.float32))   # affine dtype != scale dtype
    with pytest.raises(ValueError):
        B.linear_layernorm(X, W, a, b, workspace=T(M, N + 1, dt=torch.float32))


def test_pack_and_transpose_reject():
    with pytest.raises(ValueError):
        B.pack_signs(T(8, 48, dt=torch.int8))                        # K % 32
    with pytest.raises(ValueError):
        B.pack_signs(T(8, 64, dt=torch.int8), out=T(8, 3, dt=torch.int32))
    with pytest.raises(ValueError):
        B.transpose_signs(T(40, 2, dt=torch.int32), 40, 64)            # rows % 32
