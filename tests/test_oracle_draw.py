"""Pins for the oracle's orthogonal random features (Philox4x64-10, Box-Muller
normals, QR with a positive R diagonal, chi(d) row lengths).

The generator is checked against numpy's own Philox bit generator (a library
implementation), the normals against scipy's normal distribution, and the
features against the properties that define them (G = Q R with Q orthonormal
and R upper triangular with a positive diagonal, rows scaled by the lengths of
independent Gaussian vectors), without calling a QR routine.
"""
import math

import numpy as np
import pytest
import scipy.stats

import oracle

U64 = (1 << 64) - 1


@pytest.mark.parametrize("counter,key", [
    ((1, 0, 0, 0), (0, 0)),
    ((5, 3, 2, 1), (12345, 7)),
    ((U64, 0, 9, 0), (U64, U64)),              # word 0 at its maximum
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
])
def test_philox_matches_numpy_bit_generator(counter, key):
    # numpy's Philox increments its 256-bit counter before each block, so a
    # generator started at counter - 1 yields the block of `counter` first.
    c = list(counter)
    prev = list(c)
    prev[0] = (prev[0] - 1) & U64
    if c[0] == 0:   # borrow into word 1 (not used by the cases above)
        prev[1] = (prev[1] - 1) & U64
    g = np.random.Philox(counter=np.array(prev, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    want = [int(x) for x in g.random_raw(4)]
    assert oracle.philox4x64_10(c, key) == want


def test_normals_are_standard_normal():
    z = np.concatenate([oracle.draw_normals(11, s, 0, b, 0, 4096) for s in range(3) for b in range(3)])
    assert z.size == 36864
    ks = scipy.stats.kstest(z, "norm")
    assert ks.pvalue > 1e-4, ks
    assert abs(z.mean()) < 5 / math.sqrt(z.size)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / z.size)
    # different streams are uncorrelated
    a = oracle.draw_normals(11, 0, 0, 0, 0, 20000)
    b = oracle.draw_normals(11, 0, 0, 0, 1, 20000)
    c = oracle.draw_normals(11, 1, 0, 0, 0, 20000)
    for x, y in ((a, b), (a, c)):
        assert abs(np.corrcoef(x, y)[0, 1]) < 5 / math.sqrt(20000)
    # a prefix of a stream is the stream's prefix
    assert np.array_equal(oracle.draw_normals(11, 0, 0, 0, 0, 7), a[:7])


@pytest.mark.parametrize("H,m,d", [(2, 256, 64), (1, 100, 32), (3, 16, 16)])
def test_features_are_scaled_orthogonal_blocks(H, m, d):
    seed, step = 99, 4
    W = oracle.draw_features(seed, step, H, m, d)
    assert W.shape == (H, m, d)
    for h in range(H):
        for b in range((m + d - 1) // d):
            rows = min(d, m - b * d)
            Wb = W[h, b * d:b * d + rows]
            G = oracle.draw_normals(seed, step, h, b, 0, d * d).reshape(d, d)
            g = oracle.draw_normals(seed, step, h, b, 1, d * d).reshape(d, d)
            s = np.sqrt(np.sum(g[:rows] ** 2, axis=1))
            Q = (Wb / s[:, None]).T                      # d x rows: the first columns of Q
            np.testing.assert_allclose(Q.T @ Q, np.eye(rows), atol=1e-12)
            R = Q.T @ G                                  # rows x d: rows of R
            assert np.all(np.abs(np.tril(R[:, :rows], -1)) < 1e-10)
            assert np.all(np.diag(R[:, :rows]) > 0)
            # the rows of R reproduce G's first columns: G[:, :rows] = Q R[:, :rows]
            np.testing.assert_allclose(Q @ R[:, :rows], G[:, :rows], atol=1e-10)


def test_features_truncate_and_redraw():
    full = oracle.draw_features(5, 0, 1, 128, 64)
    cut = oracle.draw_features(5, 0, 1, 100, 64)
    assert np.array_equal(cut, full[:, :100])
    again = oracle.draw_features(5, 0, 1, 128, 64)
    assert np.array_equal(full, again)
    other = oracle.draw_features(5, 1, 1, 128, 64)
    assert np.max(np.abs(other - full)) > 0.5


def test_features_rows_have_identity_second_moment():
    # every row is marginally N(0, I_d): E[w w^T] = I
    d = 16
    acc = np.zeros((d, d))
    rows = 0
    for step in range(60):
        W = oracle.draw_features(1, step, 1, 32, d)[0]
        acc += W.T @ W
        rows += W.shape[0]
    acc /= rows
    assert np.max(np.abs(acc - np.eye(d))) < 0.12


def test_favor_estimate_is_unbiased_with_drawn_features():
    # E_W[phi(q) . phi(k)] = exp(q . k): average of the estimate over draws
    rng = np.random.default_rng(3)
    d = 8
    q = rng.standard_normal(d) * 0.4
    k = rng.standard_normal(d) * 0.4
    est = []
    for step in range(300):
        W = oracle.draw_features(2, step, 1, 16, d)[0]
        est.append(float(oracle.feature_map(q[None], W)[0] @ oracle.feature_map(k[None], W)[0]))
    assert abs(np.mean(est) / math.exp(q @ k) - 1.0) < 0.05
