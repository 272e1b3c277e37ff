"""Plain fp64 reference for FAVOR+ attention (Performer).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP path.

Every function works on float64 NumPy arrays, follows one statement of the
method written out directly, and does no blocking, fusion or reordering beyond
what that statement says (except where a docstring says the token loop is cut
into blocks only to bound memory).  Shapes: X/Q/K/V are [..., n, d] with any
leading batch/head axes; W is [m, d] (one head) or [H, m, d] broadcast over a
leading head axis that matches X's second-to-last-but-one axis.

Sources (pages on the method):
  * "Performer" paper notes (eightmm): sections Kernel Attention View,
    Normalization, FAVOR+, Standard Attention Cost.
  * "Linear Attention and the Performer" lesson (creativeworksofknowledge):
    sections The kernelization trick and Code.
  * "Performer for vision" (chipfoundryservices): How It Works (Step 1, Step 2),
    Kernel Choices, What Is Performer?.
  * "How do linear attention variants (Performer, Linformer) achieve O(n)
    complexity" (zenaique quiz page): the comparison table and the list of
    uses (the Linear Transformer's elu(x)+1 feature map).

Readings taken where the pages are silent (all stated again in the design notes):
  * phi(x) = exp(W x - |x|^2/2) / sqrt(m) with the same W for queries and keys
    (the FAVOR+ identity E[phi(q).phi(k)] = exp(q.k) uses one omega on both
    sides).  No stabiliser: this oracle computes the unshifted definition.
  * The library applies no 1/sqrt(d) temperature; inputs carry it.
  * Causal attention is inclusive: token i aggregates keys j <= i.
  * d_v = d; the denominator has no epsilon.
  * Deterministic feature maps (kind argument): "relu" is phi(x) = max(W x, 0)
    / sqrt(m) with the same random W; "elu1" is phi(x) = elu(x) + 1 applied to
    x itself (m = d, no W).  ReLU features can all be zero for a query; its
    row then has no weight at all and y is defined as 0.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "feature_map", "kv_state", "attention", "attention_causal", "decode", "attention_quadratic",
    "attention_quadratic_rows", "softmax_attention", "max_rel_err", "PHI_KINDS",
    "philox4x64_10", "draw_normals", "draw_features", "attention_backward", "attention_backward_rows",
]

PHI_KINDS = ("exp", "relu", "elu1")


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _heads_W(W: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Broadcast W ([m,d] or [H,m,d]) against X ([..., H, n, d] or [n, d])."""
    W = _f64(W)
    if W.ndim == 2:
        return W
    if W.ndim == 3:
        if X.ndim < 3 or X.shape[-3] != W.shape[0]:
            raise ValueError("W has a head axis that does not match X")
        return W
    raise ValueError("W must be [m,d] or [H,m,d]")


def feature_map(X, W, kind: str = "exp") -> np.ndarray:
    """Feature map phi, applied to each row x of X.  Returns [..., n, m].

    kind "exp": positive random features phi(x) = exp(W x - |x|^2 / 2) / sqrt(m).
      Performer notes, section FAVOR+ (positive features whose inner product
      estimates exp(q.k)); Performer for vision, Kernel Choices (exp of
      Gaussian projections keeps features positive).
    kind "relu": phi(x) = max(W x, 0) / sqrt(m).  Performer for vision, What Is
      Performer? (ReLU features) and Kernel Choices (random projections).
    kind "elu1": phi(x) = elu(x) + 1 = (x + 1 if x > 0 else exp(x)), each
      coordinate of x itself, so m = d and W is not used.  Quiz page on linear
      attention variants: the Linear Transformer's elu+1 feature map.
    """
    X = _f64(X)
    if kind == "elu1":
        return np.where(X > 0, X + 1.0, np.exp(np.minimum(X, 0.0)))
    W = _heads_W(W, X)
    m = W.shape[-2]
    if W.ndim == 2:
        proj = X @ W.T                                   # [..., n, m]
    else:
        proj = X @ np.swapaxes(W, -1, -2)               # [..., H, n, d] @ [H, d, m]
    if kind == "relu":
        return np.maximum(proj, 0.0) / math.sqrt(m)
    if kind != "exp":
        raise ValueError(f"unknown feature map {kind!r}")
    half_sq = 0.5 * np.sum(X * X, axis=-1, keepdims=True)
    return np.exp(proj - half_sq) / math.sqrt(m)


def _ratio(num, den):
    """num / den, with rows whose total weight den is 0 set to 0 (only ReLU
    features can give a query no weight at all)."""
    den = np.asarray(den)
    safe = np.where(den > 0, den, 1.0)
    return np.where(den > 0, num / safe, 0.0)


def kv_state(K, V, W, kind: str = "exp"):
    """S = Phi(K)^T V ([..., m, d]) and z = Phi(K)^T 1 ([..., m]).

    Performer notes, Kernel Attention View (the key/value summary S computed
    once) and Normalization (the summed key features in the denominator).
    """
    phiK = feature_map(K, W, kind)
    V = _f64(V)
    S = np.swapaxes(phiK, -1, -2) @ V
    z = np.sum(phiK, axis=-2)
    return S, z


def attention(Q, K, V, W, kind: str = "exp") -> np.ndarray:
    """Non-causal FAVOR+ attention y_i = phi(q_i)^T S / phi(q_i)^T z.

    Performer notes, Normalization (associative form of the normalised
    output); lesson "Linear Attention and the Performer", Code (numerator
    phi(Q)(phi(K)^T V), denominator phi(Q)(phi(K)^T 1), output their ratio).
    """
    S, z = kv_state(K, V, W, kind)
    phiQ = feature_map(Q, W, kind)
    num = phiQ @ S
    den = phiQ @ z[..., :, None]
    return _ratio(num, den)


def attention_causal(Q, K, V, W, block: int = 256, kind: str = "exp") -> np.ndarray:
    """Causal FAVOR+ attention by running prefix sums over tokens.

    Performer for vision, How It Works, Step 2 (prefix sums so each token sees
    only earlier ones) with the inclusive reading j <= i:
        S_i = S_{i-1} + phi(k_i) v_i^T,   z_i = z_{i-1} + phi(k_i),
        y_i = phi(q_i)^T S_i / phi(q_i)^T z_i.
    The token loop is cut into blocks of `block` tokens only to bound memory:
    inside a block the running sums are np.cumsum of the per-token terms, and
    the last running value carries into the next block.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    phiQ = feature_map(Q, W, kind)
    phiK = feature_map(K, W, kind)
    n = Q.shape[-2]
    lead = Q.shape[:-2]
    m = phiQ.shape[-1]
    d = V.shape[-1]
    S = np.zeros(lead + (m, d))
    z = np.zeros(lead + (m,))
    Y = np.empty(lead + (n, d))
    for s in range(0, n, block):
        e = min(n, s + block)
        outer = phiK[..., s:e, :, None] * V[..., s:e, None, :]       # [..., b, m, d]
        Srun = S[..., None, :, :] + np.cumsum(outer, axis=-3)         # S_i for i in block
        zrun = z[..., None, :] + np.cumsum(phiK[..., s:e, :], axis=-2)
        pq = phiQ[..., s:e, :]
        num = np.einsum("...bm,...bmd->...bd", pq, Srun)
        den = np.einsum("...bm,...bm->...b", pq, zrun)
        Y[..., s:e, :] = _ratio(num, den[..., None])
        S = Srun[..., -1, :, :]
        z = zrun[..., -1, :]
    return Y


def decode(Q, K, V, W, S0=None, z0=None, kind: str = "exp"):
    """Streaming (token-by-token) causal FAVOR+: the prefix sums carried as a
    state and updated one token at a time.

    Performer for vision, How It Works, Step 2 (running prefix sums, each token
    seeing only earlier ones and itself), written as the recurrence over the
    T new tokens t = 0 .. T-1, starting from the state (S0, z0) of the keys
    before them (zero state if None):
        S <- S + phi(k_t) v_t^T,   z <- z + phi(k_t),   y_t = phi(q_t)^T S / phi(q_t)^T z.
    Returns (Y [..., T, d], S [..., m, d], z [..., m]); the state is the plain
    (unshifted) one of kv_state.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    phiQ = feature_map(Q, W, kind)
    phiK = feature_map(K, W, kind)
    lead = Q.shape[:-2]
    T, d = Q.shape[-2], V.shape[-1]
    m = phiQ.shape[-1]
    S = np.zeros(lead + (m, d)) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (m,)) if z0 is None else _f64(z0).copy()
    Y = np.empty(lead + (T, d))
    for t in range(T):
        S = S + phiK[..., t, :, None] * V[..., t, None, :]
        z = z + phiK[..., t, :]
        num = np.einsum("...m,...md->...d", phiQ[..., t, :], S)
        den = np.einsum("...m,...m->...", phiQ[..., t, :], z)
        Y[..., t, :] = _ratio(num, den[..., None])
    return Y, S, z


def attention_quadratic(Q, K, V, W, causal: bool = False, kind: str = "exp") -> np.ndarray:
    """Explicit quadratic form y = (A V) / (A 1) with A = Phi(Q) Phi(K)^T.

    Performer notes, Normalization (the ratio of sums over keys before
    reassociation) and Kernel Attention View (the n x n order that FAVOR+
    avoids).  causal=True keeps A_ij only for j <= i.  Small n only.
    """
    phiQ = feature_map(Q, W, kind)
    phiK = feature_map(K, W, kind)
    A = phiQ @ np.swapaxes(phiK, -1, -2)
    if causal:
        n = A.shape[-1]
        A = A * np.tril(np.ones((n, n)))
    V = _f64(V)
    return _ratio(A @ V, np.sum(A, axis=-1, keepdims=True))


def attention_quadratic_rows(Q, K, V, W, rows, causal: bool, kind: str = "exp") -> np.ndarray:
    """Rows `rows` of the explicit quadratic form for one (batch, head) slice.

    Q, K, V are [n, d] and W is [m, d].  For each requested row i the weights
    a_j = phi(q_i)^T phi(k_j) (j <= i when causal) give y_i = sum a_j v_j / sum a_j.
    Returns [len(rows), d].  Cost is O(n m) per row, so it serves as a sampled
    check at any sequence length.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    rows = np.asarray(rows, dtype=np.int64)
    phiq = feature_map(Q[rows], W, kind)                # [r, m]
    phiK = feature_map(K, W, kind)                      # [n, m]
    out = np.empty((len(rows), V.shape[-1]))
    for t, i in enumerate(rows):
        hi = i + 1 if causal else K.shape[0]
        a = phiK[:hi] @ phiq[t]
        out[t] = _ratio(a @ V[:hi], np.sum(a))
    return out


def softmax_attention(Q, K, V, causal: bool = False) -> np.ndarray:
    """Exact attention softmax(Q K^T) V in fp64 (comparator, not a parity target).

    Performer notes, Standard Attention Cost; the 1/sqrt(d) temperature is
    already folded into Q and K by the inputs.  Row maxima are subtracted
    before exponentiating.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    L = Q @ np.swapaxes(K, -1, -2)
    if causal:
        n = L.shape[-1]
        L = np.where(np.tril(np.ones((n, n), dtype=bool)), L, -np.inf)
    L = L - np.max(L, axis=-1, keepdims=True)
    P = np.exp(L)
    return (P @ V) / np.sum(P, axis=-1, keepdims=True)


def max_rel_err(y, y_ref) -> float:
    """Error metric: max over (batch, head) slices of max|y - y_ref| / max|y_ref|.

    Outputs are convex combinations of value rows and cross zero, so an
    elementwise ratio is ill-posed; each slice is normalised by its own
    largest reference magnitude.
    """
    y = _f64(y)
    y_ref = _f64(y_ref)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {y_ref.shape}")
    if y.ndim < 2:
        y = y[None, :]
        y_ref = y_ref[None, :]
    lead = y.shape[:-2]
    a = np.abs(y - y_ref).reshape(lead + (-1,)).max(axis=-1)
    b = np.abs(y_ref).reshape(lead + (-1,)).max(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = a / b
    return float(np.max(r)) if r.size else 0.0


# ---------------------------------------------------------------------------
# Orthogonal random features drawn from a counter-based generator.
#
# Performer for vision, Kernel Choices (orthogonal features: QR of random
# projection matrices lowers the variance) and Performer notes, FAVOR+ (the
# random directions w_f).  The random numbers come from Philox4x64-10 (Salmon,
# Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", 2011),
# written here from its published definition, and Box-Muller normals.
# ---------------------------------------------------------------------------
_PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
_PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)
_U64 = (1 << 64) - 1


def philox4x64_10(counter, key):
    """One Philox4x64 block with 10 rounds: four 64-bit words from a 256-bit
    counter and a 128-bit key (Python integers).  Each round multiplies words 0
    and 2 by the two constants, mixes the high halves with words 1 and 3 and the
    key, and the key is bumped by the two Weyl constants after every round."""
    c = [int(x) & _U64 for x in counter]
    k = [int(x) & _U64 for x in key]
    for _ in range(10):
        p0 = _PHILOX_M[0] * c[0]
        p1 = _PHILOX_M[1] * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & _U64, (p0 >> 64) ^ c[3] ^ k[1], p0 & _U64]
        k = [(k[0] + _PHILOX_W[0]) & _U64, (k[1] + _PHILOX_W[1]) & _U64]
    return c


def _unit(w: int) -> float:
    """Top 53 bits of a word as a uniform number in (0, 1) (never 0 or 1)."""
    return ((w >> 11) + 0.5) * (2.0 ** -53)


def draw_normals(seed: int, step: int, head: int, block: int, kind: int, count: int) -> np.ndarray:
    """Standard normals #0 .. count-1 of the stream (head, block, kind).

    Normal j comes from the Philox block with counter (j // 4, block, head,
    kind) and key (seed, step): its words (w0, w1) and (w2, w3) give two
    Box-Muller pairs r cos(2 pi u2), r sin(2 pi u2) with r = sqrt(-2 ln u1), in
    the order w0w1-cos, w0w1-sin, w2w3-cos, w2w3-sin.
    """
    out = np.empty(count)
    for i in range((count + 3) // 4):
        w = philox4x64_10((i, block, head, kind), (seed, step))
        z = []
        for a, b in ((w[0], w[1]), (w[2], w[3])):
            r = math.sqrt(-2.0 * math.log(_unit(a)))
            t = 2.0 * math.pi * _unit(b)
            z += [r * math.cos(t), r * math.sin(t)]
        for e in range(4):
            if 4 * i + e < count:
                out[4 * i + e] = z[e]
    return out


def draw_features(seed: int, step: int, H: int, m: int, d: int) -> np.ndarray:
    """W [H, m, d] of orthogonal random features for key (seed, step).

    For each head and block b = 0 .. ceil(m/d)-1: G[r][c] = normal r*d + c of
    stream kind 0; G = Q R with R's diagonal positive (the QR that makes Q
    unique and Haar distributed); row b*d + i of W (for the rows below m) is
    s_i Q[:, i], where s_i = |g_i| and g_i holds normals i*d .. i*d + d-1 of
    stream kind 1 (a chi(d) length, the norm of an independent Gaussian
    vector).  A new step gives an independent draw (the per-call redraw).
    """
    nb = (m + d - 1) // d
    W = np.empty((H, m, d))
    for h in range(H):
        for b in range(nb):
            G = draw_normals(seed, step, h, b, 0, d * d).reshape(d, d)
            Q, R = np.linalg.qr(G)
            Q = Q * np.sign(np.diag(R))[None, :]
            g = draw_normals(seed, step, h, b, 1, d * d).reshape(d, d)
            rows = min(d, m - b * d)
            for i in range(rows):
                W[h, b * d + i] = np.linalg.norm(g[i]) * Q[:, i]
    return W


# ---------------------------------------------------------------------------
# Backward pass: dQ, dK, dV of y = phi(Q) S / phi(Q) z (non-causal) or of its
# prefix-sum form (causal), for an upstream gradient dY.
#
# The pages mention training and gradients but print no formulas; these are
# derived from the forward definitions above by the chain rule.  With
# a_i = phi(q_i), b_j = phi(k_j), den_i = a_i . z_i and y_i = a_i^T S_i / den_i
# (S_i, z_i: sums over the keys query i sees):
#   da_i = (S_i dy_i - z_i (dy_i . y_i)) / den_i
#   R_j  = sum over queries i that see key j of a_i dy_i^T / den_i     (m x d)
#   rho_j = sum over the same i of a_i (dy_i . y_i) / den_i            (m)
#   db_j = R_j v_j - rho_j,    dv_j = R_j^T b_j
# and through phi_f(x) = exp(w_f . x - |x|^2/2) / sqrt(m), whose derivative is
# phi_f(x) (w_f - x):  dx = W^T (phi(x) * dphi) - x (phi(x) . dphi).
# ---------------------------------------------------------------------------
def attention_backward(Q, K, V, W, dY, causal: bool = False):
    """(dQ, dK, dV) for upstream gradient dY, FAVOR+ features, fp64.

    Causal sums run over j <= i (the inclusive reading).  Plain loops over
    tokens in the causal case; small n only.
    """
    Q, K, V, dY = _f64(Q), _f64(K), _f64(V), _f64(dY)
    Wh = _heads_W(W, Q)
    A = feature_map(Q, W)                                  # [..., n, m]
    Bk = feature_map(K, W)
    n = Q.shape[-2]
    if causal:
        mask = np.tril(np.ones((n, n)))
    else:
        mask = np.ones((n, n))
    P = (A @ np.swapaxes(Bk, -1, -2)) * mask              # P_ij = a_i . b_j over visible keys
    den = np.sum(P, axis=-1)                               # [..., n]
    Y = (P @ V) / den[..., None]
    delta = np.sum(dY * Y, axis=-1)                        # dy_i . y_i
    # dP_ij = dy_i . (v_j - y_i) / den_i on visible pairs
    dP = ((dY @ np.swapaxes(V, -1, -2)) - delta[..., None]) / den[..., None] * mask
    dA = dP @ Bk                                           # [..., n, m]
    dB = np.swapaxes(dP, -1, -2) @ A
    dV = np.swapaxes(P / den[..., None], -1, -2) @ dY

    def through_phi(X, F, dF):
        g = F * dF                                         # phi * dphi, [..., n, m]
        if Wh.ndim == 2:
            WtG = g @ Wh
        else:
            WtG = g @ Wh                                   # [..., H, n, m] @ [H, m, d]
        return WtG - X * np.sum(g, axis=-1, keepdims=True)

    return through_phi(Q, A, dA), through_phi(K, Bk, dB), dV


def attention_backward_rows(Q, K, V, W, dY, qrows, krows, causal: bool):
    """Rows of (dQ, dK, dV) for one (batch, head) slice (Q, K, V, dY [n, d],
    W [m, d]): dQ at query rows `qrows`, dK and dV at key rows `krows`, each
    from the same definitions as attention_backward with the sums over tokens
    taken directly (O(n m d) per row), so it serves as a sampled check at any n.
    """
    Q, K, V, dY = _f64(Q), _f64(K), _f64(V), _f64(dY)
    W = _f64(W)
    n = Q.shape[0]
    A = feature_map(Q, W)                                  # [n, m]
    Bk = feature_map(K, W)
    if causal:
        S = np.cumsum(Bk[:, :, None] * V[:, None, :], axis=0)    # S_i over j <= i, [n, m, d]
        z = np.cumsum(Bk, axis=0)
    else:
        S = np.broadcast_to(Bk.T @ V, (n,) + (Bk.shape[1], V.shape[1]))
        z = np.broadcast_to(np.sum(Bk, axis=0), Bk.shape)
    den = np.einsum("im,im->i", A, z)
    Y = np.einsum("im,imd->id", A, S) / den[:, None]
    delta = np.sum(dY * Y, axis=-1)
    dQ = np.empty((len(qrows), Q.shape[1]))
    for t, i in enumerate(qrows):
        da = (S[i] @ dY[i] - z[i] * delta[i]) / den[i]
        g = A[i] * da
        dQ[t] = W.T @ g - Q[i] * np.sum(g)
    dK = np.empty((len(krows), K.shape[1]))
    dV = np.empty((len(krows), V.shape[1]))
    for t, j in enumerate(krows):
        seen = np.arange(j, n) if causal else np.arange(n)
        coef = A[seen] / den[seen, None]                   # a_i / den_i over the queries that see key j
        R = coef.T @ dY[seen]                              # [m, d]
        rho = coef.T @ delta[seen]
        db = R @ V[j] - rho
        g = Bk[j] * db
        dK[t] = W.T @ g - K[j] * np.sum(g)
        dV[t] = R.T @ Bk[j]
    return dQ, dK, dV
