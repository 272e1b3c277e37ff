"""GPU parity of the backward pass (dq, dk, dv) against the fp64 oracle,
non-causal and causal.

bf16 inputs, fp32 gradients; bar per gradient: max over (b, h) of
max|g - g_ref| / max|g_ref| <= 2e-3 (the bf16 bar).  A single token is the
degenerate case: y = v_0 whatever q and k are, so dq = dk = 0 exactly and dv =
dy; there the bound is absolute (and so for the causal first query, which sees
key 0 alone).  The causal kernels walk ranges of keys and queries in 32-token
chunks, carrying the prefix (suffix) state of the ranges before (after): the
shapes below give one range, many short ranges, and long ranges with a ragged
last chunk.  The parity cases hand the backward the
oracle's own forward output y, so that they measure the backward alone; one
case runs the GPU forward first.
"""
import numpy as np
import pytest

import favor_inputs as fi
import oracle
import oracle_pool

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import kernelized_linear_attention_favor_amd as favor  # noqa: E402

TOL = 2e-3
DEV = torch.device("cuda:0")


def gerr(g, w):
    return oracle.max_rel_err(g, w)


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=torch.bfloat16)


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=DEV)


def make(B, H, n, m, seed, scale=1.0):
    x = fi.make_inputs(fi.Config("bw", B, H, n, 64, m, "bf16", False, 64, "iid", seed), qk_scale=scale)
    rng = np.random.default_rng(seed + 1)
    dy = rng.standard_normal(x["q"].shape).astype(np.float32)
    return x, dy


def gpu_backward(x, y, dy, **kw):
    out = favor.attention_backward(bf(x["q"]), bf(x["k"]), bf(x["v"]), bf(x["W"]), f32(y), f32(dy), **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def fwd(x, causal):
    return (oracle.attention_causal if causal else oracle.attention)(x["q"], x["k"], x["v"], x["W"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("m", [64, 128, 256])
def test_backward_single_token(m, causal):
    x, dy = make(2, 2, 1, m, 299)
    y = x["v"].astype(np.float64)
    dq, dk, dv = gpu_backward(x, y, dy, causal=causal)
    # dq and dk are exact cancellations (S dy - z delta, R v - rho): what is left is
    # operand rounding (~2^-16) times |W| |v| |dy|, O(1) here; the bar is 2e-3 of a
    # gradient scale of 0.5, a floor for these O(1) inputs
    assert np.max(np.abs(dq)) < 1e-3 and np.max(np.abs(dk)) < 1e-3
    assert np.max(np.abs(dv - dy)) < 1e-4 * np.max(np.abs(dy))   # hi + lo operands: ~2^-16 relative


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("m", [64, 128, 256])
@pytest.mark.parametrize("n", [2, 31, 65, 1000, 2049])
def test_backward_matches_oracle(n, m, causal):
    x, dy = make(1, 2, n, m, 300 + n)
    got = gpu_backward(x, fwd(x, causal), dy, causal=causal)
    want = oracle.attention_backward(x["q"], x["k"], x["v"], x["W"], dy, causal=causal)
    for g, w, name in zip(got, want, ("dq", "dk", "dv")):
        assert np.all(np.isfinite(g)), name
        assert gerr(g, w) < TOL, (name, gerr(g, w))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,n,m", [(3, 40, 17, 64), (2, 64, 40, 256)])
def test_backward_many_heads_short(B, H, n, m, causal):
    # more (b, h) pairs than workgroups per pass, each shorter than one 64-token tile
    x, dy = make(B, H, n, m, 320 + H)
    got = gpu_backward(x, fwd(x, causal), dy, causal=causal)
    want = oracle.attention_backward(x["q"], x["k"], x["v"], x["W"], dy, causal=causal)
    for g, w, name in zip(got, want, ("dq", "dk", "dv")):
        assert np.all(np.isfinite(g)), name
        assert gerr(g, w) < TOL, (name, gerr(g, w))


@pytest.mark.parametrize("B,H,n,m", [(4, 8, 1000, 128), (2, 4, 3000, 64), (8, 8, 777, 256)])
def test_backward_causal_long_ranges(B, H, n, m):
    # many (b, h): few ranges per head, each several chunks long, the last one ragged
    x, dy = make(B, H, n, m, 310 + n)
    got = gpu_backward(x, fwd(x, True), dy, causal=True)
    want = oracle.attention_backward(x["q"], x["k"], x["v"], x["W"], dy, causal=True)
    for g, w, name in zip(got, want, ("dq", "dk", "dv")):
        assert gerr(g, w) < TOL, (name, gerr(g, w))
    # query 0 sees key 0 alone (y_0 = v_0): its dq cancels
    assert np.max(np.abs(got[0][:, :, 0])) < 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_backward_C2_shape_and_large_inputs(causal):
    for scale, seed in ((1.0, 2), (2.0, 3)):
        x, dy = make(1, 8, 1024, 256, seed, scale)
        got = gpu_backward(x, fwd(x, causal), dy, causal=causal)
        want = oracle.attention_backward(x["q"], x["k"], x["v"], x["W"], dy, causal=causal)
        for g, w in zip(got, want):
            assert gerr(g, w) < TOL


@pytest.mark.parametrize("causal", [False, True])
def test_backward_far_features(causal):
    """Features far above the first 32: W's first 32 rows are zero and the others long, so
    some query's exponents lie ~90 (log2) above its first feature tile's largest. The
    non-causal query pass shifts by that tile's maximum and redoes the tile with the exact
    maximum when a weight would exceed 2^64; the keys' exponents spread ~53 below their
    largest."""
    x, dy = make(1, 2, 200, 64, 77)
    rng = np.random.default_rng(5)
    W = x["W"].astype(np.float64)
    W[:, :32] = 0.0
    W[:, 32:] *= 8.0 / np.sqrt(64)
    x["W"] = fi.round_bf16(W.astype(np.float32))
    x["q"] = fi.round_bf16((rng.standard_normal(x["q"].shape) * 1.5).astype(np.float32))
    x["k"] = fi.round_bf16((rng.standard_normal(x["k"].shape) * 0.5).astype(np.float32))
    got = gpu_backward(x, fwd(x, causal), dy, causal=causal)
    want = oracle.attention_backward(x["q"], x["k"], x["v"], x["W"], dy, causal=causal)
    for g, w, name in zip(got, want, ("dq", "dk", "dv")):
        assert np.all(np.isfinite(g)), name
        assert gerr(g, w) < TOL, (name, gerr(g, w))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_C5_low_rank(causal):
    """The vision stand-in's low-rank q, k (m = 128, H = 12) at n = 1024."""
    x = fi.make_inputs(fi.config("C5", B=1, n=1024))
    dy = np.random.default_rng(13).standard_normal(x["q"].shape).astype(np.float32)
    got = gpu_backward(x, fwd(x, causal), dy, causal=causal)
    want = oracle.attention_backward(x["q"], x["k"], x["v"], x["W"], dy, causal=causal)
    for g, w, name in zip(got, want, ("dq", "dk", "dv")):
        assert np.all(np.isfinite(g)), name
        assert gerr(g, w) < TOL, (name, gerr(g, w))


def _range_span(n, BH, causal):
    """Token span of the backward's key/query ranges (the kernels' own plan:
    about 512 ranges over B*H non-causal, 256 causal, each a multiple of 64)."""
    s = min(max(1, ((256 if causal else 512) + BH - 1) // BH), (n + 63) // 64)
    return ((n + s - 1) // s + 63) // 64 * 64


C3_SLICES = ((0, 0), (1, 3), (2, 5), (3, 7))


def _c3_rows(n, span, seed):
    """Rows to check in one slice: both sides of every range boundary, the
    first and last tokens, 32-token chunk edges inside the first range, and
    random rows, at least 64 in all."""
    rng = np.random.default_rng(seed)
    edges = [r for k in range(1, (n + span - 1) // span) for r in (k * span - 1, k * span)]
    rows = set(edges) | {0, 1, 31, 32, 63, 64, n - 2, n - 1}
    target = max(64, len(rows) + 24)
    while len(rows) < target:
        rows.add(int(rng.integers(0, n)))
    return np.array(sorted(rows))


def _c3_backward(causal):
    cfg = fi.config("C3")
    x = fi.make_inputs(cfg)
    dy = np.random.default_rng(8).standard_normal(x["q"].shape).astype(np.float32)
    t = {k: bf(v) for k, v in x.items()}
    y_gpu = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=causal)
    # the checked slices get the oracle's forward output, so that the bar measures the backward
    yref = oracle_pool.reference(x, causal=causal, slices=list(C3_SLICES))
    y_or = y_gpu.clone()
    for b, h in C3_SLICES:
        y_or[b, h] = torch.from_numpy(yref[b, h].astype(np.float32)).to(DEV)
    g_or = favor.attention_backward(t["q"], t["k"], t["v"], t["W"], y_or, f32(dy), causal=causal)
    g_gpu = favor.attention_backward(t["q"], t["k"], t["v"], t["W"], y_gpu, f32(dy), causal=causal)
    torch.cuda.synchronize()
    g_or = [a.cpu().numpy() for a in g_or]
    g_gpu = [a.cpu().numpy() for a in g_gpu]
    span = _range_span(cfg.n, cfg.B * cfg.H, causal)
    rows = {bh: _c3_rows(cfg.n, span, 9 + 3 * bh[0] + bh[1]) for bh in C3_SLICES}
    want = oracle_pool.backward_rows(x, dy, causal, rows)
    return g_or, g_gpu, rows, want


def _rows_err(g, bh, r, w):
    # normalised by the largest reference gradient among the checked rows: never larger than
    # the slice's own maximum, so this bar is at least as strict as the per-slice metric
    return float(np.max(np.abs(g[bh[0], bh[1]][r] - w)) / max(np.max(np.abs(w)), 1e-30))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_C3_shape_rows(causal):
    """B=4, H=8, n=16384, m=256, the benchmark's shape: dq, dk, dv on >= 64 rows of
    each of 4 slices (both sides of every range boundary), given the oracle's y, at
    the bf16 bar.  The same rows from the GPU forward's y are reported beside
    (end to end) and must meet the bar too."""
    g_or, g_gpu, rows, want = _c3_backward(causal)
    for g in g_or + g_gpu:
        assert np.all(np.isfinite(g))
    worst_or, worst_e2e = 0.0, 0.0
    for bh, r in rows.items():
        for k, name in enumerate(("dq", "dk", "dv")):
            e = _rows_err(g_or[k], bh, r, want[bh][k])
            e2 = _rows_err(g_gpu[k], bh, r, want[bh][k])
            worst_or, worst_e2e = max(worst_or, e), max(worst_e2e, e2)
            assert e < TOL, (bh, name, e)
    print(f"C3 backward causal={causal}: worst {worst_or:.3e} (oracle y), {worst_e2e:.3e} (GPU forward y)")
    assert worst_e2e < TOL


@pytest.mark.parametrize("causal", [False, True])
def test_backward_end_to_end_and_determinism(causal):
    x, dy = make(2, 4, 3000, 256, 11)
    t = {k: bf(v) for k, v in x.items()}
    y = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=causal)
    a = favor.attention_backward(t["q"], t["k"], t["v"], t["W"], y, f32(dy), causal=causal)
    nb = favor._lib.favor_backward_workspace_bytes(2, 4, 3000, 64, 256, int(causal))
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    b = favor.attention_backward(t["q"], t["k"], t["v"], t["W"], y, f32(dy), causal=causal, workspace=ws)
    c = favor.attention_backward(t["q"], t["k"], t["v"], t["W"], y, f32(dy), causal=causal, workspace=ws)
    torch.cuda.synchronize()
    for u, w, z in zip(a, b, c):
        assert torch.equal(u, w) and torch.equal(u, z)
    want = oracle.attention_backward(x["q"], x["k"], x["v"], x["W"], dy, causal=causal)
    for g, w in zip(a, want):
        assert gerr(g.cpu().numpy(), w) < TOL


def test_backward_workspace_too_small_raises():
    x, dy = make(1, 2, 300, 64, 12)
    nb = favor._lib.favor_backward_workspace_bytes(1, 2, 300, 64, 64, 1)
    ws = torch.zeros(nb - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(favor.FavorError):
        gpu_backward(x, fwd(x, True), dy, causal=True, workspace=ws)
