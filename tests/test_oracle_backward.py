"""Pins for the oracle's backward pass (dQ, dK, dV).

The hand-derived gradients are checked against torch's automatic
differentiation of an fp64 forward written as the explicit quadratic form, and
against central finite differences of the oracle's own forward; the sampled-row
form against the full form.
"""
import numpy as np
import pytest
import torch

import oracle


def _inputs(seed, B=2, H=2, n=24, d=8, m=16, scale=1.0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, n, d)) * d ** -0.25 * scale
    K = rng.standard_normal((B, H, n, d)) * d ** -0.25 * scale
    V = rng.standard_normal((B, H, n, d))
    W = rng.standard_normal((H, m, d))
    dY = rng.standard_normal((B, H, n, d))
    return Q, K, V, W, dY


def _torch_forward(Q, K, V, W, causal):
    """y = (A V) / (A 1), A_ij = phi(q_i) . phi(k_j) (j <= i when causal), in torch."""
    m = W.shape[-2]
    Wt = W.transpose(-1, -2).unsqueeze(0)                  # [1, H, d, m]

    def phi(X):
        return torch.exp(X @ Wt - 0.5 * (X * X).sum(-1, keepdim=True)) / m ** 0.5

    A = phi(Q) @ phi(K).transpose(-1, -2)
    if causal:
        n = A.shape[-1]
        A = A * torch.tril(torch.ones(n, n, dtype=A.dtype))
    return (A @ V) / A.sum(-1, keepdim=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [1.0, 2.0])
def test_backward_matches_autograd(causal, scale):
    Q, K, V, W, dY = _inputs(3 + int(causal), scale=scale)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    y = _torch_forward(tq, tk, tv, torch.tensor(W), causal)
    gq, gk, gv = torch.autograd.grad(y, (tq, tk, tv), grad_outputs=torch.tensor(dY))
    dQ, dK, dV = oracle.attention_backward(Q, K, V, W, dY, causal=causal)
    for got, want in ((dQ, gq), (dK, gk), (dV, gv)):
        want = want.numpy()
        assert np.max(np.abs(got - want)) <= 1e-10 * np.max(np.abs(want))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    Q, K, V, W, dY = _inputs(5, B=1, H=1, n=6, d=4, m=8)
    f = oracle.attention_causal if causal else oracle.attention
    loss = lambda q, k, v: float(np.sum(f(q, k, v, W) * dY))
    dQ, dK, dV = oracle.attention_backward(Q, K, V, W, dY, causal=causal)
    h = 1e-6
    for X, G, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        for idx in [(0, 0, 0, 0), (0, 0, 3, 2), (0, 0, 5, 1)]:
            args_p = [Q.copy(), K.copy(), V.copy()]
            args_m = [Q.copy(), K.copy(), V.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(num - G[idx]) <= 1e-6 * max(1.0, abs(num)), (which, idx, num, G[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_backward_rows_match_full(causal):
    Q, K, V, W, dY = _inputs(7, B=1, H=1, n=40)
    dQ, dK, dV = oracle.attention_backward(Q, K, V, W, dY, causal=causal)
    rows = [0, 1, 17, 39]
    q, k, v = oracle.attention_backward_rows(Q[0, 0], K[0, 0], V[0, 0], W[0], dY[0, 0], rows, rows, causal)
    np.testing.assert_allclose(q, dQ[0, 0][rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(k, dK[0, 0][rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(v, dV[0, 0][rows], rtol=1e-10, atol=1e-12)


def test_backward_value_gradient_is_a_weighted_sum_of_dy():
    # dV_j = sum_i P_ij dy_i / den_i: with dY = 1 for every entry, every key's
    # dV row is the total attention weight it receives (non-causal)
    Q, K, V, W, _ = _inputs(9, B=1, H=1, n=10)
    dY = np.ones_like(V)
    _, _, dV = oracle.attention_backward(Q, K, V, W, dY)
    A = oracle.feature_map(Q, W)[0, 0] @ oracle.feature_map(K, W)[0, 0].T
    w = (A / A.sum(axis=1, keepdims=True)).sum(axis=0)
    np.testing.assert_allclose(dV[0, 0], np.repeat(w[:, None], V.shape[-1], axis=1), rtol=1e-12)
    assert abs(dV.sum() / V.shape[-1] - 10.0) < 1e-10     # the weights of each query sum to 1
