"""GPU parity of the deterministic feature maps (ReLU features of W, elu(x)+1)
against the fp64 oracle, non-causal and causal.

bf16 inputs, fp32 output; bar: max over (b, h) of max|y - y_ref| / max|y_ref|
<= 2e-3 (the bf16 bar).  The kernels carry phi, S and the causal chunk matrix
as bf16 hi + lo pairs, so the measured errors sit far below it.
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
KINDS = [("relu", 64), ("relu", 128), ("relu", 256), ("elu1", 64)]


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=torch.bfloat16)


def run(x, kind, causal, **kw):
    W = None if kind == "elu1" else bf(x["W"])
    y = favor.attention(bf(x["q"]), bf(x["k"]), bf(x["v"]), W, causal=causal, phi=kind, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def ref(x, kind, causal):
    W = None if kind == "elu1" else x["W"]
    f = oracle.attention_causal if causal else oracle.attention
    return f(x["q"], x["k"], x["v"], W, kind=kind)


def inputs(B, H, n, m, seed, **kw):
    return fi.make_inputs(fi.Config("phi", B, H, n, 64, m, "bf16", False, 64, "iid", seed), **kw)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind,m", KINDS)
@pytest.mark.parametrize("n", [1, 31, 33, 64, 65, 100, 1000, 2049])
def test_phi_ragged(kind, m, causal, n):
    x = inputs(1, 2, n, m, 900 + n)
    y = run(x, kind, causal)
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, ref(x, kind, causal)) < TOL


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind,m", [("relu", 256), ("elu1", 64)])
def test_phi_C2_shape(kind, m, causal):
    x = inputs(1, 8, 1024, m, 2)
    y = run(x, kind, causal)
    err = oracle.max_rel_err(y, ref(x, kind, causal))
    assert err < 1e-4, err   # hi + lo operands: far below the bf16 bar


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind,m", [("relu", 256), ("elu1", 64)])
def test_phi_C3_shape_slices(kind, m, causal):
    """B=4, H=8, n=16384: the launch the benchmark times; whole (b, h) slices
    (every row) against the oracle, normalised by the oracle's own maximum."""
    x = inputs(4, 8, 16384, m, 3)
    y = run(x, kind, causal)
    assert np.all(np.isfinite(y))
    xx = dict(x)
    if kind == "elu1":
        xx["W"] = None
    slices = [(0, 0), (1, 5), (2, 2), (3, 7)]
    r = oracle_pool.reference(xx, causal=causal, kind=kind, slices=slices)
    errs = oracle_pool.slice_errors(y, r, slices)
    assert max(errs.values()) < TOL, errs


@pytest.mark.parametrize("kind,m", [("relu", 128), ("elu1", 64)])
@pytest.mark.parametrize("scale", [2.0, 4.0])
def test_phi_large_inputs(kind, m, scale):
    x = inputs(2, 2, 700, m, 40, qk_scale=scale)
    for causal in (False, True):
        y = run(x, kind, causal)
        assert np.all(np.isfinite(y))
        assert oracle.max_rel_err(y, ref(x, kind, causal)) < TOL


def test_phi_C5_low_rank():
    x = fi.make_inputs(fi.config("C5", B=2, n=1024))
    for kind in ("relu", "elu1"):
        xx = dict(x)
        if kind == "elu1":
            xx["W"] = None
        for causal in (False, True):
            W = None if kind == "elu1" else bf(x["W"])
            y = favor.attention(bf(x["q"]), bf(x["k"]), bf(x["v"]), W, causal=causal, phi=kind)
            torch.cuda.synchronize()
            r = (oracle.attention_causal if causal else oracle.attention)(x["q"], x["k"], x["v"], xx["W"], kind=kind)
            assert oracle.max_rel_err(y.cpu().numpy(), r) < TOL


def test_relu_rows_without_weight_are_zero():
    # all-positive W and negative queries: those queries have no feature, so y = 0
    x = inputs(1, 2, 300, 128, 41)
    x["W"] = np.abs(x["W"])
    x["q"][:, :, 10] = -np.abs(x["q"][:, :, 10])
    x["q"][:, :, 200] = -np.abs(x["q"][:, :, 200])
    x = {k: fi.round_bf16(v) for k, v in x.items()}
    for causal in (False, True):
        y = run(x, "relu", causal)
        assert np.all(np.isfinite(y))
        assert np.all(y[:, :, 10] == 0) and np.all(y[:, :, 200] == 0)
        assert oracle.max_rel_err(y, ref(x, "relu", causal)) < TOL


def test_elu1_constant_keys_give_prefix_means():
    # k = 0: every key feature is 1, so y_i is the mean of v over the keys it sees
    x = inputs(1, 2, 500, 64, 42)
    x["k"][:] = 0.0
    v = x["v"].astype(np.float64)
    yc = run(x, "elu1", True)
    y = run(x, "elu1", False)
    pre = np.cumsum(v, axis=2) / np.arange(1, 501)[None, None, :, None]
    assert oracle.max_rel_err(yc, pre) < 1e-5
    assert oracle.max_rel_err(y, np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)) < 1e-5


@pytest.mark.parametrize("kind,m", [("relu", 256), ("elu1", 64)])
def test_phi_workspace_determinism_and_first_row(kind, m):
    x = inputs(2, 4, 3000, m, 43)
    for causal in (False, True):
        a = run(x, kind, causal)
        b = run(x, kind, causal)
        ws = favor.Workspace(2, 4, 3000, 64, m, causal=causal, phi=kind)
        c = run(x, kind, causal, workspace=ws)
        d = run(x, kind, causal, workspace=ws)
        assert np.array_equal(a, b) and np.array_equal(a, c) and np.array_equal(a, d)
    # causal row 0 sees only key 0: y_0 = v_0 whenever phi(q_0).phi(k_0) > 0
    y = run(x, kind, True)
    W = None if kind == "elu1" else x["W"]
    pq = oracle.feature_map(x["q"][:, :, :1], W, kind)
    pk = oracle.feature_map(x["k"][:, :, :1], W, kind)
    w0 = np.sum(pq * pk, axis=-1)[..., 0]
    for b in range(2):
        for h in range(4):
            if w0[b, h] > 0:
                assert np.max(np.abs(y[b, h, 0] - x["v"][b, h, 0])) < 1e-5


def test_phi_errors_raise():
    x = inputs(1, 1, 16, 64, 44)
    with pytest.raises(ValueError):
        favor.attention(bf(x["q"]), bf(x["k"]), bf(x["v"]), bf(x["W"]), phi="softplus")
    with pytest.raises(ValueError):   # ReLU features need W
        favor.attention(bf(x["q"]), bf(x["k"]), bf(x["v"]), None, phi="relu")
    with pytest.raises(favor.FavorError):   # elu+1 needs m = d: the library refuses W with m = 128
        favor.attention(bf(x["q"]), bf(x["k"]), bf(x["v"]), bf(np.zeros((1, 128, 64), np.float32)), phi="elu1")
