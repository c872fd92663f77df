"""CPU tests: the fp64 oracle against its pins, and planted mistakes against the pins."""
import numpy as np
import pytest

import oracle as O
from bit_weight_linear_amd import workloads as W
from tests import oracle_pins as P


# ---------------------------------------------------------------- the oracle passes every pin
def test_pack_pins():
    assert P.pin_pack_patterns(O.pack_signs, O.unpack_signs) == []


@pytest.mark.parametrize("pin", P.ONEBIT_PINS, ids=lambda p: p.__name__)
def test_onebit_pins(pin):
    assert pin(O.onebit_linear) == []


@pytest.mark.parametrize("pin", P.DBF_PINS, ids=lambda p: p.__name__)
def test_dbf_pins(pin):
    assert pin(O.dbf_linear) == []


def test_sign_of_zero_and_negative_zero():
    S = O.sign_pm1(np.array([[0.0, -0.0, -1e-30, 1e-30, -3.0, 2.0]]))
    assert S.tolist() == [[1, 1, -1, 1, -1, 1]]
    # packing reads the sign the same way
    Z = np.zeros((1, 32))
    Z[0, 3] = -0.0
    Z[0, 4] = -1e-30
    assert O.pack_signs(Z)[0, 0] == (1 << 4)


def test_dbf_stage1_is_onebit_with_m_as_output_scale():
    c = W.dbf_case(3, 64, 32, 48, seed=2)
    T1 = O.dbf_stage1(c.X, c.S2, c.b, c.m)
    chain = (c.X * c.b[None, :]) @ c.S2.T.astype(np.float64) * c.m[None, :]
    scale = (np.abs(c.X) @ np.abs(c.b))[:, None] * np.abs(c.m)[None, :]
    assert (np.abs(T1 - chain) <= 1e-12 * scale).all()


def test_error_scales_bound_outputs():
    c = W.onebit_case(4, 256, 96, kind="signed_scales", seed=3)
    Y = O.onebit_linear(c.X, c.W_sign, c.a, c.b)
    assert (np.abs(Y) <= O.onebit_error_scale(c.X, c.a, c.b) * (1 + 1e-12)).all()
    d = W.dbf_case(3, 64, 32, 40, seed=4)
    Yd = O.dbf_linear(d.X, d.S1, d.S2, d.a, d.m, d.b)
    assert (np.abs(Yd) <= O.dbf_error_scale(d.X, d.b, d.m, d.a) * (1 + 1e-12)).all()


def test_max_normalised_error():
    S = np.array([[1.0, 2.0, 0.0]])
    assert O.max_normalised_error([[1.5, 2.0, 0.0]], [[1.0, 2.0, 0.0]], S) == 0.5
    assert O.max_normalised_error([[1.0, 2.0, 1.0]], [[1.0, 2.0, 0.0]], S) == np.inf


# ---------------------------------------------------------------- rank-1 helpers
def test_power_iteration_matches_lapack_and_lemma1():
    """OneBit page lemma 1: σ1(|W|) >= σ1(W); power iteration agrees with LAPACK's SVD."""
    rng = np.random.default_rng(0)
    for t in range(200):
        shape = [(4, 8), (8, 8), (16, 16)][t % 3]
        A = rng.standard_normal(shape)
        s_lapack = np.linalg.svd(A, compute_uv=False)[0]
        s_abs_lapack = np.linalg.svd(np.abs(A), compute_uv=False)[0]
        s = O.power_iteration_sigma1(A)
        s_abs = O.power_iteration_sigma1(np.abs(A))
        assert abs(s - s_lapack) <= 1e-9 * s_lapack
        assert abs(s_abs - s_abs_lapack) <= 1e-9 * s_abs_lapack
        assert s_abs >= s * (1 - 1e-12)


def test_rank1_is_eckart_young_optimal():
    """The rank-1 truncation error equals the sum of the trailing squared singular values."""
    rng = np.random.default_rng(1)
    A = rng.standard_normal((12, 9))
    s, u, v = O.rank1_power(A)
    err = np.linalg.norm(A - s * np.outer(u, v)) ** 2
    sv = np.linalg.svd(A, compute_uv=False)
    assert abs(err - (sv[1:] ** 2).sum()) <= 1e-9 * (sv ** 2).sum()


def test_svid_proposition2():
    """OneBit page proposition 2: the SVID error is no larger than the plain rank-1 error,
    and ||W||_F = || |W| ||_F."""
    rng = np.random.default_rng(2)
    for _ in range(60):
        Wm = rng.standard_normal((8, 6))
        sign, a, b = O.svid(Wm)
        assert (a >= 0).all() and (b >= 0).all()
        assert np.array_equal(sign, O.sign_pm1(Wm))
        e_svid = np.linalg.norm(Wm - sign * np.outer(a, b)) ** 2
        s, u, v = O.rank1_power(Wm)
        e_rank1 = np.linalg.norm(Wm - s * np.outer(u, v)) ** 2
        assert e_svid <= e_rank1 * (1 + 1e-9)
        assert abs(np.linalg.norm(Wm) - np.linalg.norm(np.abs(Wm))) <= 1e-12 * np.linalg.norm(Wm)


def test_svid_recovers_planted_rank1_magnitudes():
    rng = np.random.default_rng(3)
    a0 = np.abs(rng.standard_normal(10)) + 0.5
    b0 = np.abs(rng.standard_normal(7)) + 0.5
    S = W.random_signs(rng, (10, 7))
    sign, a, b = O.svid(S * np.outer(a0, b0))
    assert np.array_equal(sign, S)
    assert np.allclose(np.outer(a, b), np.outer(a0, b0), rtol=1e-10, atol=0)


# ---------------------------------------------------------------- generators
def test_workload_generators_are_deterministic_and_typed():
    for i in (1, 5):
        c1, c2 = W.workload(i), W.workload(i)
        assert np.array_equal(c1.X, c2.X)
        assert np.array_equal(c1.a, c2.a) and np.array_equal(c1.b, c2.b)
    c = W.workload(1)
    assert c.X.shape == (4, 512) and c.W_sign.shape == (512, 512)
    assert np.array_equal(W.round_to(c.X, "f32"), c.X)
    d = W.workload(5)
    assert d.S2.shape == (3072, 4096) and d.S1.shape == (4096, 3072)
    assert np.array_equal(W.round_to(d.m, "f16"), d.m)
    # outlier structure: six fixed channels carry the large values
    c3 = W.onebit_case(16, 4096, 64, seed=0)
    big = np.abs(c3.X).max(axis=0)
    assert (np.sort(big)[-6:] > 20).all() and np.sort(big)[-7] < 10


def test_round_to_bf16_is_rne():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -20)])
    assert W.round_to(x, "bf16").tolist() == [1.0, 1.0, 1 + 2 ** -6, -(1 + 2 ** -7)]


# ---------------------------------------------------------------- planted mistakes are caught
def _dense(S, a, b):
    return np.asarray(S, float) * np.asarray(a, float)[:, None] * np.asarray(b, float)[None, :]


ONEBIT_MUTANTS = {
    "no_transpose": lambda X, S, a, b: np.asarray(X, float) @ _dense(S, a, b),
    "sign_flip": lambda X, S, a, b: O.onebit_linear(X, -np.asarray(S), a, b),
    "drop_a": lambda X, S, a, b: O.onebit_linear(X, S, np.ones_like(np.asarray(a, float)), b),
    "drop_b": lambda X, S, a, b: O.onebit_linear(X, S, a, np.ones_like(np.asarray(b, float))),
    "swap_a_b": lambda X, S, a, b: np.asarray(X, float) @ (np.asarray(S, float) * np.asarray(b, float)[:, None] * np.asarray(a, float)[None, :]).T,
    "shifted_k": lambda X, S, a, b: O.onebit_linear(X, np.roll(np.asarray(S), 1, axis=1), a, b),
    "abs_x": lambda X, S, a, b: O.onebit_linear(np.abs(np.asarray(X, float)), S, a, b),
    "dropped_last_k": lambda X, S, a, b: O.onebit_linear(np.asarray(X, float)[:, :-1], np.asarray(S)[:, :-1], a, np.asarray(b, float)[:-1]),
}


@pytest.mark.parametrize("name", sorted(ONEBIT_MUTANTS))
def test_onebit_mutants_fail_some_pin(name):
    assert P.run(P.ONEBIT_PINS, ONEBIT_MUTANTS[name]) != [], f"mutant {name} passed every pin"


PACK_MUTANTS = {
    "msb_first": (lambda S: O.pack_signs(np.asarray(S).reshape(len(S), -1, 32)[:, :, ::-1].reshape(len(S), -1)),
                  O.unpack_signs),
    "inverted_polarity": (lambda S: ~O.pack_signs(S), O.unpack_signs),
    "reversed_words": (lambda S: O.pack_signs(S)[:, ::-1].copy(),
                       lambda P_, K: O.unpack_signs(np.asarray(P_)[:, ::-1].copy(), K)),
    "unpack_polarity": (O.pack_signs, lambda P_, K: -O.unpack_signs(P_, K)),
}


@pytest.mark.parametrize("name", sorted(PACK_MUTANTS))
def test_pack_mutants_fail_some_pin(name):
    pack, unpack = PACK_MUTANTS[name]
    assert P.pin_pack_patterns(pack, unpack) != [], f"mutant {name} passed"


DBF_MUTANTS = {
    "drop_m": lambda X, S1, S2, a, m, b: O.dbf_linear(X, S1, S2, a, np.ones_like(np.asarray(m, float)), b),
    "drop_a": lambda X, S1, S2, a, m, b: O.dbf_linear(X, S1, S2, np.ones_like(np.asarray(a, float)), m, b),
    "drop_b": lambda X, S1, S2, a, m, b: O.dbf_linear(X, S1, S2, a, m, np.ones_like(np.asarray(b, float))),
    "flip_S2": lambda X, S1, S2, a, m, b: O.dbf_linear(X, S1, -np.asarray(S2), a, m, b),
    "S1_transposed": lambda X, S1, S2, a, m, b: np.asarray(X, float) @ ((np.asarray(a, float)[:, None] * np.asarray(S1, float).T * np.asarray(m, float)[None, :]) @ (np.asarray(S2, float) * np.asarray(b, float)[None, :])).T,
    "a_b_swapped": lambda X, S1, S2, a, m, b: O.dbf_linear(X, S1, S2, b, m, a),
}


@pytest.mark.parametrize("name", sorted(DBF_MUTANTS))
def test_dbf_mutants_fail_some_pin(name):
    assert P.run(P.DBF_PINS, DBF_MUTANTS[name]) != [], f"mutant {name} passed every pin"


# ---------------------------------------------------------------- backward and transposed packing
@pytest.mark.parametrize("pin", P.BACKWARD_PINS, ids=lambda p: p.__name__)
def test_backward_pins(pin):
    assert pin(O.onebit_backward) == []


def test_transpose_signs_is_the_transposed_packing():
    rng = np.random.default_rng(41)
    S = W.random_signs(rng, (96, 160))
    P_ = O.pack_signs(S)
    PT = O.transpose_signs(P_, 96, 160)
    assert PT.shape == (160, 3) and PT.dtype == np.uint32
    assert np.array_equal(O.unpack_signs(PT, 96), S.T)
    # bit j of PT[k, w] is the sign of S[32w + j, k]
    k, w, j = 7, 2, 5
    assert ((int(PT[k, w]) >> j) & 1) == (1 if S[32 * w + j, k] < 0 else 0)
    assert np.array_equal(O.transpose_signs(PT, 160, 96), P_)


def test_backward_error_scales_bound_gradients():
    rng = np.random.default_rng(43)
    X, dY = rng.standard_normal((4, 64)), rng.standard_normal((4, 32))
    S = W.random_signs(rng, (32, 64))
    a, b = rng.standard_normal(32), rng.standard_normal(64)
    dX, da, db = O.onebit_backward(X, S, a, b, dY)
    sdx, sda, sdb = O.backward_error_scales(X, a, b, dY)
    assert np.all(np.abs(dX) <= sdx + 1e-12) and np.all(np.abs(da) <= sda + 1e-12)
    assert np.all(np.abs(db) <= sdb + 1e-12)


def _bw(X, S, a, b, dY, **over):
    args = dict(a=a, b=b)
    args.update(over)
    return O.onebit_backward(X, S, args["a"], args["b"], dY)


BACKWARD_MUTANTS = {
    "dX_without_scales": lambda X, S, a, b, dY: (np.asarray(dY, float) @ np.asarray(S, float),
                                                 *_bw(X, S, a, b, dY)[1:]),
    "dX_missing_b": lambda X, S, a, b, dY: (_bw(X, S, a, b, dY, b=np.ones(len(b)))[0], *_bw(X, S, a, b, dY)[1:]),
    "da_missing_b": lambda X, S, a, b, dY: (_bw(X, S, a, b, dY)[0], _bw(X, S, a, b, dY, b=np.ones(len(b)))[1],
                                            _bw(X, S, a, b, dY)[2]),
    "db_missing_a": lambda X, S, a, b, dY: (*_bw(X, S, a, b, dY)[:2], _bw(X, S, a, b, dY, a=np.ones(len(a)))[2]),
    "sign_flip": lambda X, S, a, b, dY: O.onebit_backward(X, -np.asarray(S), a, b, dY),
}


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutants_fail_some_pin(name):
    assert P.run(P.BACKWARD_PINS, BACKWARD_MUTANTS[name]) != [], f"mutant {name} passed every pin"


# ---------------------------------------------------------------- LayerNorm after the layer
@pytest.mark.parametrize("pin", P.LAYERNORM_PINS, ids=lambda p: p.__name__)
def test_layernorm_pins(pin):
    assert pin(O.layernorm_rows) == []


def _ln_unbiased(Y, eps=1e-5, gamma=None, beta=None):
    Y = np.asarray(Y, float)
    mu = Y.mean(1, keepdims=True)
    var = ((Y - mu) ** 2).sum(1, keepdims=True) / (Y.shape[1] - 1)
    return (Y - mu) / np.sqrt(var + eps)


LAYERNORM_MUTANTS = {
    "unbiased_variance": _ln_unbiased,
    "eps_outside_sqrt": lambda Y, eps=1e-5, gamma=None, beta=None: (
        (np.asarray(Y, float) - np.asarray(Y, float).mean(1, keepdims=True))
        / (np.asarray(Y, float).std(1, keepdims=True) + eps)),
    "no_centering": lambda Y, eps=1e-5, gamma=None, beta=None: (
        np.asarray(Y, float) / np.sqrt(np.asarray(Y, float).var(1, keepdims=True) + eps)),
    "gamma_ignored": lambda Y, eps=1e-5, gamma=None, beta=None: O.layernorm_rows(Y, eps, None, beta),
}


@pytest.mark.parametrize("name", sorted(LAYERNORM_MUTANTS))
def test_layernorm_mutants_fail_some_pin(name):
    assert P.run(P.LAYERNORM_PINS, LAYERNORM_MUTANTS[name]) != [], f"mutant {name} passed every pin"
