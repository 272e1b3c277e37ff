"""Pins for the oracle's deterministic feature maps (kind "relu" and "elu1").

Each check reaches the same numbers by an independent route: a library elu,
hand-worked values, an identity of the ReLU (relu(a) - relu(-a) = a) checked
against plain dot products, the explicit quadratic form, closed forms for
constant features, and the positive homogeneity of ReLU features.
"""
import math

import numpy as np
import pytest
import torch

import oracle

KINDS = ("relu", "elu1")


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(seed, shape=(2, 3, 40, 8), m=24):
    rng = _rng(seed)
    B, H, n, d = shape
    Q = rng.standard_normal(shape) * d ** -0.25
    K = rng.standard_normal(shape) * d ** -0.25
    V = rng.standard_normal(shape)
    W = rng.standard_normal((H, m, d))
    return Q, K, V, W


# ------------------------------------------------------------------ elu + 1
def test_elu1_matches_library_elu():
    X = _rng(1).standard_normal((3, 50, 16)) * 2.0
    want = torch.nn.functional.elu(torch.from_numpy(X)).numpy() + 1.0
    got = oracle.feature_map(X, None, "elu1")
    assert got.shape == X.shape
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=1e-15)


def test_elu1_hand_worked():
    x = np.array([[-1.0, 0.0, 2.0, -3.5]])
    want = [math.exp(-1.0), 1.0, 3.0, math.exp(-3.5)]
    got = oracle.feature_map(x, None, "elu1")[0]
    for g, w in zip(got, want):
        assert abs(g - w) <= 1e-15 * w
    assert np.all(oracle.feature_map(_rng(2).standard_normal((10, 6)) * 5, None, "elu1") > 0)


def test_elu1_zero_keys_give_value_means():
    # K = 0: every key feature is 1, so each query weights every key equally:
    # non-causal y_i = mean_j v_j, causal y_i = mean_{j<=i} v_j.
    rng = _rng(3)
    n, d = 30, 8
    Q = rng.standard_normal((n, d))
    K = np.zeros((n, d))
    V = rng.standard_normal((n, d))
    y = oracle.attention(Q, K, V, None, kind="elu1")
    yc = oracle.attention_causal(Q, K, V, None, block=7, kind="elu1")
    for i in range(n):
        for c in range(d):
            all_mean = sum(float(V[j, c]) for j in range(n)) / n
            pre_mean = sum(float(V[j, c]) for j in range(i + 1)) / (i + 1)
            assert abs(y[i, c] - all_mean) <= 1e-13
            assert abs(yc[i, c] - pre_mean) <= 1e-13


# --------------------------------------------------------------------- relu
def test_relu_hand_worked():
    W = np.array([[1.0, 2.0], [-1.0, 0.5]])
    # x = (1, 1): w1.x = 3, w2.x = -0.5 -> (3, 0) / sqrt(2)
    got = oracle.feature_map(np.array([[1.0, 1.0]]), W, "relu")[0]
    assert abs(got[0] - 3.0 / math.sqrt(2)) <= 1e-15 and got[1] == 0.0
    # x = (0.5, -1): both projections negative -> no feature
    assert np.all(oracle.feature_map(np.array([[0.5, -1.0]]), W, "relu") == 0.0)


def test_relu_sign_identity_against_plain_dot_products():
    # relu(a) - relu(-a) = a, so phi(x) - phi(-x) = W x / sqrt(m), and for each
    # feature at most one of phi(x), phi(-x) is nonzero.
    rng = _rng(4)
    m, d = 12, 5
    W = rng.standard_normal((m, d))
    X = rng.standard_normal((7, d))
    P, N = oracle.feature_map(X, W, "relu"), oracle.feature_map(-X, W, "relu")
    for i in range(7):
        for f in range(m):
            dot = sum(float(W[f, k]) * float(X[i, k]) for k in range(d))
            assert abs((P[i, f] - N[i, f]) - dot / math.sqrt(m)) <= 1e-14
            assert P[i, f] >= 0 and N[i, f] >= 0 and P[i, f] * N[i, f] == 0


def test_relu_positive_scaling_invariance():
    # ReLU features are positively homogeneous: scaling queries or keys by a
    # positive constant scales numerator and denominator alike.
    Q, K, V, W = _inputs(5)
    y = oracle.attention(Q, K, V, W, kind="relu")
    yc = oracle.attention_causal(Q, K, V, W, kind="relu")
    assert oracle.max_rel_err(oracle.attention(3.0 * Q, 0.25 * K, V, W, kind="relu"), y) < 1e-13
    assert oracle.max_rel_err(oracle.attention_causal(0.5 * Q, 7.0 * K, V, W, kind="relu"), yc) < 1e-13
    # the exp features are not homogeneous: the same scaling changes them
    ye = oracle.attention(Q, K, V, W)
    assert oracle.max_rel_err(oracle.attention(3.0 * Q, 0.25 * K, V, W), ye) > 1e-3


def test_relu_row_without_weight_is_zero():
    # All-positive W and an all-negative query: every projection is negative, the
    # query has no feature, its row carries no weight and y = 0 (the reading).
    rng = _rng(6)
    n, d, m = 12, 4, 8
    W = np.abs(rng.standard_normal((m, d))) + 0.1
    Q = rng.standard_normal((n, d))
    Q[5] = -np.abs(Q[5]) - 0.1
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    for y in (oracle.attention(Q, K, V, W, kind="relu"),
              oracle.attention_causal(Q, K, V, W, kind="relu"),
              oracle.attention_quadratic(Q, K, V, W, causal=True, kind="relu")):
        assert np.all(y[5] == 0.0)
        assert np.all(np.isfinite(y))


# ------------------------------------------------- both kinds: associativity
@pytest.mark.parametrize("kind", KINDS)
def test_phi_attention_matches_quadratic_form(kind):
    Q, K, V, W = _inputs(7 + len(kind))
    if kind == "elu1":
        W = None
    q = oracle.attention_quadratic(Q, K, V, W, kind=kind)
    assert oracle.max_rel_err(oracle.attention(Q, K, V, W, kind=kind), q) < 1e-12
    qc = oracle.attention_quadratic(Q, K, V, W, causal=True, kind=kind)
    assert oracle.max_rel_err(oracle.attention_causal(Q, K, V, W, block=9, kind=kind), qc) < 1e-12
    rows = [0, 3, 17, 39]
    for causal, ref in ((False, q), (True, qc)):
        got = oracle.attention_quadratic_rows(Q[1, 2], K[1, 2], V[1, 2], None if W is None else W[2], rows,
                                              causal, kind=kind)
        assert oracle.max_rel_err(got, ref[1, 2][rows]) < 1e-12


@pytest.mark.parametrize("kind", KINDS)
def test_phi_decode_matches_causal(kind):
    Q, K, V, W = _inputs(9, shape=(1, 2, 25, 8))
    if kind == "elu1":
        W = None
    y, S, z = oracle.decode(Q, K, V, W, kind=kind)
    assert oracle.max_rel_err(y, oracle.attention_causal(Q, K, V, W, kind=kind)) < 1e-12
    Sk, zk = oracle.kv_state(K, V, W, kind)
    assert oracle.max_rel_err(S, Sk) < 1e-12
    np.testing.assert_allclose(z, zk, rtol=1e-12)


def test_unknown_kind_is_rejected():
    with pytest.raises(ValueError):
        oracle.feature_map(np.zeros((2, 3)), np.zeros((4, 3)), "softplus")
