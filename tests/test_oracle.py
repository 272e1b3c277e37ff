"""Pins for the fp64 oracle: closed forms, quadrature, brute force and invariants.

None of these checks retypes the oracle's own formulas: each compares an
oracle function with an independent route to the same number (hand-derived
closed forms evaluated with math.exp, Gauss-Hermite quadrature of the FAVOR+
expectation, the explicit quadratic form, a library softmax attention, or a
property the mathematics fixes).
"""
import math

import numpy as np
import pytest
import torch

import favor_inputs as fi
import oracle


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# feature map phi(x) = exp(W x - |x|^2/2) / sqrt(m)
# --------------------------------------------------------------------------
def test_feature_map_hand_worked():
    # d = 2, m = 2.  w_1 = (1, 2), w_2 = (-1, 0.5); x = (0.5, -1).
    # w_1.x = -1.5, w_2.x = -1.0, |x|^2/2 = 0.625.
    W = np.array([[1.0, 2.0], [-1.0, 0.5]])
    x = np.array([[0.5, -1.0]])
    want = [math.exp(-1.5 - 0.625) / math.sqrt(2), math.exp(-1.0 - 0.625) / math.sqrt(2)]
    got = oracle.feature_map(x, W)[0]
    assert got.shape == (2,)
    for g, w in zip(got, want):
        assert abs(g - w) <= 1e-15 * w


def test_feature_map_scaled_identity_closed_form():
    # W = s I (m = d): phi_f(x) = exp(s x_f - |x|^2/2) / sqrt(d), evaluated elementwise.
    d, s = 8, 1.7
    rng = _rng(11)
    X = rng.standard_normal((5, d))
    got = oracle.feature_map(X, s * np.eye(d))
    for i in range(5):
        sq = sum(float(v) * float(v) for v in X[i])
        for f in range(d):
            want = math.exp(s * float(X[i, f]) - 0.5 * sq) / math.sqrt(d)
            assert abs(got[i, f] - want) <= 2e-15 * want
    # x = 0 gives 1/sqrt(m) for every feature, whatever W is.
    Wr = rng.standard_normal((12, d))
    assert np.allclose(oracle.feature_map(np.zeros((3, d)), Wr), 1 / math.sqrt(12), rtol=0, atol=1e-16)


def test_feature_map_head_broadcast():
    rng = _rng(3)
    X = rng.standard_normal((2, 3, 4, 5))          # [B, H, n, d]
    W = rng.standard_normal((3, 7, 5))             # [H, m, d]
    got = oracle.feature_map(X, W)
    assert got.shape == (2, 3, 4, 7)
    for b in range(2):
        for h in range(3):
            np.testing.assert_allclose(got[b, h], oracle.feature_map(X[b, h], W[h]), rtol=1e-15)


def _gh_plane_features(q, k, N):
    """W whose rows are t_a e1 + t_b e2 on an N x N Gauss-Hermite grid of the
    plane spanned by q and k, plus the matching probability weights."""
    t, w = np.polynomial.hermite_e.hermegauss(N)
    w = w / math.sqrt(2 * math.pi)
    e1 = q / np.linalg.norm(q)
    r = k - (k @ e1) * e1
    e2 = r / np.linalg.norm(r)
    rows = (t[:, None, None] * e1[None, None, :] + t[None, :, None] * e2[None, None, :]).reshape(N * N, -1)
    weights = (w[:, None] * w[None, :]).reshape(-1)
    return rows, weights


@pytest.mark.parametrize("seed,scale", [(1, 0.5), (2, 1.0), (3, 1.5)])
def test_unbiased_by_quadrature(seed, scale):
    """E_w[phi_w(q) phi_w(k)] = exp(q.k) for w ~ N(0, I_d) (FAVOR+ identity).

    The expectation depends only on w's projection onto span(q, k), a standard
    2-D Gaussian, so a Gauss-Hermite product rule evaluates it to machine
    precision.  Each grid node is one feature row; m * phi(q)_f phi(k)_f undoes
    the 1/sqrt(m) on both sides.
    """
    rng = _rng(seed)
    d = 16
    q = rng.standard_normal(d) * scale / 2
    k = rng.standard_normal(d) * scale / 2
    rows, wts = _gh_plane_features(q, k, 48)
    m = rows.shape[0]
    pq = oracle.feature_map(q[None, :], rows)[0]
    pk = oracle.feature_map(k[None, :], rows)[0]
    est = float(np.sum(wts * m * pq * pk))
    assert abs(est / math.exp(q @ k) - 1) < 1e-11


def test_single_feature_mean_is_one_by_quadrature():
    # E_w[exp(w.x - |x|^2/2)] = 1: the -|x|^2/2 term is exactly the Gaussian
    # moment-generating-function normaliser.
    rng = _rng(5)
    x = rng.standard_normal(10) * 0.8
    t, w = np.polynomial.hermite_e.hermegauss(60)
    w = w / math.sqrt(2 * math.pi)
    rows = t[:, None] * (x / np.linalg.norm(x))[None, :]
    phi = oracle.feature_map(x[None, :], rows)[0] * math.sqrt(len(t))
    assert abs(float(np.sum(w * phi)) - 1.0) < 1e-12


def test_unbiased_monte_carlo_orthogonal_W():
    """Monte Carlo over orthogonal W at small norms: mean / exp(q.k) within 4 s.e."""
    d = m = 16
    T = 20000
    rng = _rng(7)
    q = rng.standard_normal(d)
    q *= 0.6 / np.linalg.norm(q)
    k = rng.standard_normal(d)
    k *= 0.6 / np.linalg.norm(k)
    W = fi.orthogonal_W(np.random.default_rng(8), T, m, d)          # T independent draws
    pq = oracle.feature_map(np.broadcast_to(q, (T, 1, d)), W)[:, 0, :]
    pk = oracle.feature_map(np.broadcast_to(k, (T, 1, d)), W)[:, 0, :]
    est = np.sum(pq * pk, axis=1) / math.exp(q @ k)
    se = est.std(ddof=1) / math.sqrt(T)
    assert abs(est.mean() - 1.0) < 4 * se
    assert se < 5e-3


def test_orthogonal_lowers_variance():
    """Orthogonal features give lower estimator variance than iid ones."""
    d = m = 16
    T = 20000
    rng = _rng(9)
    q = rng.standard_normal(d)
    q *= 0.6 / np.linalg.norm(q)
    k = rng.standard_normal(d)
    k *= 0.6 / np.linalg.norm(k)
    Wo = fi.orthogonal_W(np.random.default_rng(10), T, m, d)
    Wi = fi.iid_W(np.random.default_rng(11), T, m, d)

    def est(W):
        pq = oracle.feature_map(np.broadcast_to(q, (T, 1, d)), W)[:, 0, :]
        pk = oracle.feature_map(np.broadcast_to(k, (T, 1, d)), W)[:, 0, :]
        return np.sum(pq * pk, axis=1)

    vo, vi = est(Wo).var(), est(Wi).var()
    # iid theory: Var = exp(2 q.k) (exp(|q+k|^2) - 1) / m
    theory = math.exp(2 * q @ k) * (math.exp(np.sum((q + k) ** 2)) - 1) / m
    assert abs(vi / theory - 1) < 0.1
    assert vo < 0.92 * vi


# --------------------------------------------------------------------------
# aggregation: linear form, quadratic form, causal prefix sums
# --------------------------------------------------------------------------
def test_tiny_attention_closed_form_cosh():
    # d = 1, m = 2, W = [[1], [-1]]:
    #   phi(q).phi(k) = (e^{q+k} + e^{-q-k}) e^{-(q^2+k^2)/2} / 2 = cosh(q+k) e^{-(q^2+k^2)/2}
    # so y_i = sum_j cosh(q_i+k_j) e^{-k_j^2/2} v_j / sum_j cosh(q_i+k_j) e^{-k_j^2/2}.
    q = [0.3, -0.7, 1.1]
    k = [0.5, -0.2, 0.9]
    v = [1.0, -2.0, 0.25]
    W = np.array([[1.0], [-1.0]])
    Q = np.array(q)[:, None]
    K = np.array(k)[:, None]
    V = np.array(v)[:, None]
    y = oracle.attention(Q, K, V, W)[:, 0]
    yc = oracle.attention_causal(Q, K, V, W)[:, 0]
    for i in range(3):
        a = [math.cosh(q[i] + k[j]) * math.exp(-k[j] ** 2 / 2) for j in range(3)]
        want = sum(a[j] * v[j] for j in range(3)) / sum(a)
        wantc = sum(a[j] * v[j] for j in range(i + 1)) / sum(a[: i + 1])
        assert abs(y[i] - want) < 1e-15
        assert abs(yc[i] - wantc) < 1e-15


def test_single_feature_cancels_query():
    # m = 1: phi(q_i) is a per-row scalar that cancels, y_i = sum_j phi(k_j) v_j / sum_j phi(k_j).
    rng = _rng(12)
    Q, K, V = rng.standard_normal((3, 20, 4))
    w = rng.standard_normal((1, 4))
    a = [math.exp(float(w[0] @ K[j]) - 0.5 * float(K[j] @ K[j])) for j in range(20)]
    want = sum(a[j] * V[j] for j in range(20)) / sum(a)
    y = oracle.attention(Q, K, V, w)
    assert np.max(np.abs(y - want[None, :])) < 1e-14


@pytest.mark.parametrize("n,d,m", [(1, 4, 8), (7, 4, 8), (64, 16, 32), (33, 8, 24)])
def test_linear_equals_quadratic(n, d, m):
    """(Phi(Q) Phi(K)^T) V / rowsum == Phi(Q)(Phi(K)^T V) / Phi(Q)(Phi(K)^T 1)."""
    rng = _rng(n * 131 + d)
    Q = rng.standard_normal((2, 3, n, d)) * d ** -0.25
    K = rng.standard_normal((2, 3, n, d)) * d ** -0.25
    V = rng.standard_normal((2, 3, n, d))
    W = fi.orthogonal_W(rng, 3, m, d)
    y = oracle.attention(Q, K, V, W)
    yq = oracle.attention_quadratic(Q, K, V, W)
    assert oracle.max_rel_err(y, yq) < 1e-12


def test_linear_equals_quadratic_C1():
    x = fi.make_inputs(fi.config("C1"))
    y = oracle.attention(x["q"], x["k"], x["v"], x["W"])
    yq = oracle.attention_quadratic(x["q"], x["k"], x["v"], x["W"])
    assert oracle.max_rel_err(y, yq) < 1e-12


@pytest.mark.parametrize("block", [1, 7, 64, 256, 1000])
def test_causal_prefix_equals_masked_quadratic(block):
    rng = _rng(21)
    n, d, m = 96, 8, 16
    Q = rng.standard_normal((1, 2, n, d)) * d ** -0.25
    K = rng.standard_normal((1, 2, n, d)) * d ** -0.25
    V = rng.standard_normal((1, 2, n, d))
    W = fi.orthogonal_W(rng, 2, m, d)
    yc = oracle.attention_causal(Q, K, V, W, block=block)
    yq = oracle.attention_quadratic(Q, K, V, W, causal=True)
    assert oracle.max_rel_err(yc, yq) < 1e-12


def test_causal_prefix_512_C4_shape():
    """Causal prefix sums vs the masked quadratic on a 512-token prefix of the
    long-sequence causal workload (d = 64, m = 256)."""
    cfg = fi.config("C4", B=1, H=2, n=512)
    x = fi.make_inputs(cfg)
    yc = oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])
    yq = oracle.attention_quadratic(x["q"], x["k"], x["v"], x["W"], causal=True)
    assert oracle.max_rel_err(yc, yq) < 1e-12


def test_quadratic_rows_match_full():
    rng = _rng(31)
    n, d, m = 50, 8, 16
    Q, K, V = rng.standard_normal((3, n, d)) * 0.5
    W = fi.orthogonal_W(rng, 1, m, d)[0]
    rows = [0, 1, 17, 49]
    for causal in (False, True):
        full = oracle.attention_quadratic(Q, K, V, W, causal=causal)[rows]
        part = oracle.attention_quadratic_rows(Q, K, V, W, rows, causal=causal)
        assert np.max(np.abs(full - part)) < 1e-13


# --------------------------------------------------------------------------
# invariants of the normalised form
# --------------------------------------------------------------------------
def _case(seed, n=40, d=8, m=16, B=1, H=2):
    rng = _rng(seed)
    Q = rng.standard_normal((B, H, n, d)) * d ** -0.25
    K = rng.standard_normal((B, H, n, d)) * d ** -0.25
    V = rng.standard_normal((B, H, n, d))
    W = fi.orthogonal_W(rng, H, m, d)
    return Q, K, V, W


@pytest.mark.parametrize("causal", [False, True])
def test_convexity(causal):
    """Positive weights: every output coordinate lies within the range of the
    values it averages (Performer notes: positive feature map)."""
    Q, K, V, W = _case(41)
    f = oracle.attention_causal if causal else oracle.attention
    y = f(Q, K, V, W)
    n = V.shape[-2]
    for i in range(n):
        Vs = V[..., : i + 1, :] if causal else V
        assert np.all(y[..., i, :] >= Vs.min(axis=-2) - 1e-13)
        assert np.all(y[..., i, :] <= Vs.max(axis=-2) + 1e-13)


def test_constant_values_and_identical_keys():
    Q, K, V, W = _case(42)
    c = np.arange(V.shape[-1], dtype=np.float64) - 2.5
    Vc = np.broadcast_to(c, V.shape)
    assert np.max(np.abs(oracle.attention(Q, K, Vc, W) - c)) < 1e-14
    assert np.max(np.abs(oracle.attention_causal(Q, K, Vc, W) - c)) < 1e-14
    Ks = np.broadcast_to(K[..., :1, :], K.shape)
    y = oracle.attention(Q, Ks, V, W)
    assert np.max(np.abs(y - V.mean(axis=-2, keepdims=True))) < 1e-13
    yc = oracle.attention_causal(Q, Ks, V, W)
    run_mean = np.cumsum(V, axis=-2) / np.arange(1, V.shape[-2] + 1)[:, None]
    assert np.max(np.abs(yc - run_mean)) < 1e-13


def test_single_token_and_first_row():
    Q, K, V, W = _case(43, n=1)
    assert np.max(np.abs(oracle.attention(Q, K, V, W) - V)) < 1e-15
    Q, K, V, W = _case(44)
    yc = oracle.attention_causal(Q, K, V, W)
    assert np.max(np.abs(yc[..., 0, :] - V[..., 0, :])) < 1e-15
    y = oracle.attention(Q, K, V, W)
    assert np.max(np.abs(yc[..., -1, :] - y[..., -1, :])) < 1e-13


def test_linearity_and_permutations():
    Q, K, V, W = _case(45)
    rng = _rng(46)
    V2 = rng.standard_normal(V.shape)
    a, b = 0.7, -1.3
    lhs = oracle.attention(Q, K, a * V + b * V2, W)
    rhs = a * oracle.attention(Q, K, V, W) + b * oracle.attention(Q, K, V2, W)
    assert np.max(np.abs(lhs - rhs)) < 1e-13
    perm = rng.permutation(K.shape[-2])
    y = oracle.attention(Q, K, V, W)
    yp = oracle.attention(Q, K[..., perm, :], V[..., perm, :], W)
    assert np.max(np.abs(y - yp)) < 1e-13
    yq = oracle.attention(Q[..., perm, :], K, V, W)
    assert np.max(np.abs(yq - y[..., perm, :])) < 1e-13


def test_row_and_key_shifts_cancel():
    """Per-query-row factors on phi(q) and one common factor on every phi(k)
    cancel in the ratio: the identity that lets a stabilised kernel subtract
    maxima before exponentiating."""
    Q, K, V, W = _case(47, B=1, H=1)
    Q, K, V, W = Q[0, 0], K[0, 0], V[0, 0], W[0]
    y = oracle.attention(Q, K, V, W)
    rng = _rng(48)
    row = np.exp(rng.standard_normal((Q.shape[0], 1)) * 5)
    S, z = oracle.kv_state(K, V, W)
    c = math.exp(-3.7)
    phiQ = oracle.feature_map(Q, W) * row
    y2 = (phiQ @ (c * S)) / (phiQ @ (c * z))[:, None]
    assert np.max(np.abs(y - y2)) < 1e-13


def test_kv_state_definition_bruteforce():
    rng = _rng(49)
    n, d, m = 6, 3, 4
    K, V = rng.standard_normal((2, n, d))
    W = rng.standard_normal((m, d))
    S, z = oracle.kv_state(K, V, W)
    for f in range(m):
        zf = 0.0
        for j in range(n):
            p = math.exp(sum(W[f, t] * K[j, t] for t in range(d)) - 0.5 * sum(K[j, t] ** 2 for t in range(d))) / math.sqrt(m)
            zf += p
        assert abs(z[f] - zf) < 1e-14 * max(1.0, zf)
    for f in range(m):
        for c in range(d):
            want = 0.0
            for j in range(n):
                p = math.exp(sum(W[f, t] * K[j, t] for t in range(d)) - 0.5 * sum(K[j, t] ** 2 for t in range(d))) / math.sqrt(m)
                want += p * V[j, c]
            assert abs(S[f, c] - want) < 1e-14 * max(1.0, abs(want))


# --------------------------------------------------------------------------
# softmax comparator and convergence in m
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_matches_library(causal):
    rng = _rng(51)
    Q, K, V = rng.standard_normal((3, 2, 3, 37, 8))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V), is_causal=causal, scale=1.0
    ).numpy()
    got = oracle.softmax_attention(Q, K, V, causal=causal)
    assert np.max(np.abs(got - want)) < 1e-13


def test_error_vs_softmax_shrinks_with_m():
    """Well-conditioned regime (|q|^2 about 1): the relative error against exact
    softmax falls roughly like m^-1/2 (Performer notes, FAVOR+)."""
    d, n = 16, 64
    ms = [16, 64, 256, 1024]
    errs = []
    for m in ms:
        e = []
        for s in range(8):
            rng = _rng(1000 + s)
            Q = rng.standard_normal((n, d)) * d ** -0.5
            K = rng.standard_normal((n, d)) * d ** -0.5
            V = rng.standard_normal((n, d))
            W = fi.orthogonal_W(np.random.default_rng(5000 + 97 * s + m), 1, m, d)[0]
            y = oracle.attention(Q, K, V, W)
            ys = oracle.softmax_attention(Q, K, V)
            e.append(np.linalg.norm(y - ys) / np.linalg.norm(ys))
        errs.append(float(np.mean(e)))
    assert all(a > b for a, b in zip(errs, errs[1:]))
    slope = np.polyfit(np.log(ms), np.log(errs), 1)[0]
    assert -0.7 < slope < -0.3


# --------------------------------------------------------------------------
# error metric
# --------------------------------------------------------------------------
def test_max_rel_err_metric():
    ref = np.zeros((2, 3, 4, 5))
    ref[..., 0, 0] = 2.0
    ref[1, 2, 3, 4] = -8.0
    y = ref.copy()
    y[0, 1, 2, 3] += 0.02        # slice (0,1): max|ref| = 2 -> 0.01
    y[1, 2, 0, 1] += 0.04        # slice (1,2): max|ref| = 8 -> 0.005
    assert abs(oracle.max_rel_err(y, ref) - 0.01) < 1e-15
    with pytest.raises(ValueError):
        oracle.max_rel_err(y[..., :3], ref)


# ---------------------------------------------------------------- streaming decode
def _small(seed, B=1, H=2, n=70, d=8, m=16, scale=1.0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, n, d)) * scale * d ** -0.25
    K = rng.standard_normal((B, H, n, d)) * scale * d ** -0.25
    V = rng.standard_normal((B, H, n, d))
    W = rng.standard_normal((H, m, d))
    return Q, K, V, W


def test_decode_from_empty_equals_causal_prefix_sums():
    Q, K, V, W = _small(11)
    Y, S, z = oracle.decode(Q, K, V, W)
    np.testing.assert_allclose(Y, oracle.attention_causal(Q, K, V, W, block=16), rtol=1e-12, atol=1e-13)
    Sk, zk = oracle.kv_state(K, V, W)
    np.testing.assert_allclose(S, Sk, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(z, zk, rtol=1e-12)


def test_decode_continues_a_prefix_state():
    Q, K, V, W = _small(12, n=50)
    p = 31
    S0, z0 = oracle.kv_state(K[..., :p, :], V[..., :p, :], W)
    Y, S, z = oracle.decode(Q[..., p:, :], K[..., p:, :], V[..., p:, :], W, S0, z0)
    full = oracle.attention_quadratic(Q, K, V, W, causal=True)   # independent masked form
    np.testing.assert_allclose(Y, full[..., p:, :], rtol=1e-11, atol=1e-12)
    Sk, zk = oracle.kv_state(K, V, W)
    np.testing.assert_allclose(S, Sk, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(z, zk, rtol=1e-12)


def test_decode_first_token_and_constant_values():
    Q, K, V, W = _small(13, n=20)
    Y, _, _ = oracle.decode(Q, K, V, W)
    np.testing.assert_allclose(Y[..., 0, :], V[..., 0, :], rtol=1e-12, atol=1e-13)   # y_0 = v_0
    Vc = np.broadcast_to(np.linspace(-2.0, 3.0, V.shape[-1]), V.shape)
    Yc, _, _ = oracle.decode(Q, K, Vc, W)
    np.testing.assert_allclose(Yc, Vc, rtol=1e-12, atol=1e-12)


def test_decode_state_is_additive():
    # the state of a sequence is the sum of its parts' states (associativity of the prefix sums)
    Q, K, V, W = _small(14, n=40)
    _, Sa, za = oracle.decode(Q[..., :17, :], K[..., :17, :], V[..., :17, :], W)
    _, Sb, zb = oracle.decode(Q[..., 17:, :], K[..., 17:, :], V[..., 17:, :], W)
    _, S, z = oracle.decode(Q, K, V, W)
    np.testing.assert_allclose(Sa + Sb, S, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(za + zb, z, rtol=1e-12)
