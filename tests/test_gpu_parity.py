"""GPU parity: libfavor's HIP path against the fp64 oracle on identical inputs.

Tolerances (max over (b, h) of max|y - y_ref| / max|y_ref|):
  bf16 inputs, fp32 accumulation : 2e-3
  fp32 inputs                    : 1e-5
  feature map (elementwise rel.) : 1e-5
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

TOL_BF16 = 2e-3
TOL_F32 = 1e-5
DEV = torch.device("cuda:0")


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=dtype)


def run(x, dtype, causal=False, **kw):
    t = {k: dev(v, dtype) for k, v in x.items()}
    y = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=causal, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ----------------------------------------------------------------- feature map
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,n,d,m", [(1, 1, 1, 64, 64), (2, 3, 37, 64, 256), (1, 2, 100, 32, 48),
                                       (1, 1, 65, 16, 130)])
def test_feature_map(dtype, B, H, n, d, m):
    cfg = fi.Config("fm", B, H, n, d, m, dtype, False, 64, "iid", 7)
    x = fi.make_inputs(cfg)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    phi = favor.feature_map(dev(x["q"], td), dev(x["W"], td))
    torch.cuda.synchronize()
    ref = oracle.feature_map(x["q"], x["W"])
    rel = np.max(np.abs(phi.cpu().numpy() - ref) / ref)
    assert rel < 1e-5


# ---------------------------------------------------------------- fp32 path
def test_f32_C1_noncausal_and_causal():
    x = fi.make_inputs(fi.config("C1"))
    y = run(x, torch.float32)
    assert oracle.max_rel_err(y, oracle.attention(x["q"], x["k"], x["v"], x["W"])) < TOL_F32
    yc = run(x, torch.float32, causal=True)
    assert oracle.max_rel_err(yc, oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])) < TOL_F32


@pytest.mark.parametrize("B,H,n,d,m", [(1, 1, 1, 32, 64), (2, 2, 37, 16, 48), (1, 3, 300, 64, 256),
                                       (1, 1, 129, 128, 128)])
def test_f32_shapes(B, H, n, d, m):
    cfg = fi.Config("f32", B, H, n, d, m, "f32", False, 64, "iid", 11)
    x = fi.make_inputs(cfg)
    y = run(x, torch.float32)
    assert oracle.max_rel_err(y, oracle.attention(x["q"], x["k"], x["v"], x["W"])) < TOL_F32
    yc = run(x, torch.float32, causal=True)
    assert oracle.max_rel_err(yc, oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])) < TOL_F32


# ---------------------------------------------------------------- bf16 path
def test_bf16_C2_against_oracle_and_softmax():
    x = fi.make_inputs(fi.config("C2"))
    y = run(x, torch.bfloat16)
    ref = oracle.attention(x["q"], x["k"], x["v"], x["W"])
    err = oracle.max_rel_err(y, ref)
    sm = oracle.softmax_attention(x["q"], x["k"], x["v"])
    div = np.linalg.norm(y - sm) / np.linalg.norm(sm)
    print(f"C2 bf16: err vs oracle {err:.3e}; relative Frobenius divergence from softmax {div:.3f}")
    assert err < TOL_BF16


@pytest.mark.parametrize("n", [1, 7, 31, 32, 33, 64, 65, 100, 1000, 4097])
@pytest.mark.parametrize("m", [64, 128, 256])
def test_bf16_ragged(n, m):
    cfg = fi.Config("rag", 1, 2, n, 64, m, "bf16", False, 64, "iid", 100 + n)
    x = fi.make_inputs(cfg)
    y = run(x, torch.bfloat16)
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, oracle.attention(x["q"], x["k"], x["v"], x["W"])) < TOL_BF16


def _full_noncausal(cfg_name):
    cfg = fi.config(cfg_name)
    x = fi.make_inputs(cfg)
    y = run(x, torch.bfloat16)
    assert np.all(np.isfinite(y))
    ref = oracle_pool.reference(x, causal=False)
    errs = oracle_pool.slice_errors(y, ref, [(b, h) for b in range(cfg.B) for h in range(cfg.H)])
    worst = max(errs.values())
    print(f"{cfg_name} bf16 err {worst:.3e} over {len(errs)} slices")
    return worst


@pytest.mark.parametrize("B,H,n,d,m", [(10, 13, 1000, 64, 256), (3, 100, 300, 64, 128), (20, 55, 70, 64, 48),
                                       (6, 100, 100, 32, 64)])
def test_bf16_single_key_range(B, H, n, d, m):
    """Many (b, h) pairs: each has one key range, so the state pass writes the
    output kernel's inputs itself (no merge), including masked features (m = 48
    in 64-feature tiles) and d = 32; the output grid cuts each sequence into the
    query runs that fill whole rounds of workgroups.  Ragged n."""
    cfg = fi.Config("single", B, H, n, d, m, "bf16", False, 64, "iid", 7 + n + m)
    x = fi.make_inputs(cfg)
    y = run(x, torch.bfloat16)
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, oracle.attention(x["q"], x["k"], x["v"], x["W"])) < TOL_BF16


@pytest.mark.parametrize("m", [256, 512])
@pytest.mark.parametrize("n", [1, 31, 65, 300, 4097])
def test_bf16_output_stays_in_bounds(n, m):
    """The output kernel's last tile runs past the sequence end; nothing may
    land there: the rows after `out` in a larger buffer keep their sentinel.
    (m = 512 takes the two-query-tile form.)"""
    cfg = fi.Config("bounds", 1, 1, n, 64, m, "bf16", False, 64, "iid", 900 + n + m)
    x = fi.make_inputs(cfg)
    t = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    pad = 512 * 64
    big = torch.full((n * 64 + pad,), 12345.0, dtype=torch.float32, device=DEV)
    out = big[: n * 64].view(1, 1, n, 64)
    favor.attention(t["q"], t["k"], t["v"], t["W"], causal=False, out=out)
    torch.cuda.synchronize()
    assert bool((big[n * 64:] == 12345.0).all())
    y = out.cpu().numpy()
    assert oracle.max_rel_err(y, oracle.attention(x["q"], x["k"], x["v"], x["W"])) < TOL_BF16


def test_bf16_C3_full():
    assert _full_noncausal("C3") < TOL_BF16


def test_bf16_C5_full():
    assert _full_noncausal("C5") < TOL_BF16


@pytest.mark.parametrize("scale", [2.0, 4.0])
def test_bf16_stress_large_norms(scale):
    """Q, K scaled up: exponents far outside fp32 exp range without shifts."""
    cfg = fi.config("C2", H=4)
    x = fi.make_inputs(cfg, qk_scale=scale)
    y = run(x, torch.bfloat16)
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, oracle.attention(x["q"], x["k"], x["v"], x["W"])) < TOL_BF16


def test_bf16_overflow_fallback():
    """First keys of the range tiny next to later ones: the first-tile shift
    would overflow, so the kernel must take its recompute path."""
    cfg = fi.config("C2", H=2, n=512)
    x = fi.make_inputs(cfg)
    k = x["k"].astype(np.float64)
    k[:, :, :64, :] *= 12.0      # huge norms -> exponents around -700 for the first tile
    x["k"] = fi.round_bf16(k)
    y = run(x, torch.bfloat16)
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, oracle.attention(x["q"], x["k"], x["v"], x["W"])) < TOL_BF16


def test_bf16_convexity_determinism_workspace():
    cfg = fi.config("C2", H=4, n=2000)
    x = fi.make_inputs(cfg)
    t = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    y1 = favor.attention(t["q"], t["k"], t["v"], t["W"])
    y2 = favor.attention(t["q"], t["k"], t["v"], t["W"])
    ws = favor.Workspace(1, 4, 2000, 64, 256)
    y3 = favor.attention(t["q"], t["k"], t["v"], t["W"], workspace=ws)
    y4 = favor.attention(t["q"], t["k"], t["v"], t["W"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3) and torch.equal(y1, y4)
    y = y1.cpu().numpy()
    v = x["v"]
    assert np.all(y <= v.max(axis=-2, keepdims=True) + 1e-6)
    assert np.all(y >= v.min(axis=-2, keepdims=True) - 1e-6)


def test_bf16_constant_values():
    cfg = fi.config("C2", H=2, n=300)
    x = fi.make_inputs(cfg)
    x["v"] = np.broadcast_to(fi.round_bf16(np.linspace(-3, 3, 64)), x["v"].shape).copy()
    y = run(x, torch.bfloat16)
    assert np.max(np.abs(y - x["v"])) < 3 * 2 ** -11


# ---------------------------------------------------------------- bf16 causal
@pytest.mark.parametrize("n", [1, 7, 31, 64, 65, 100, 1000, 4097])
@pytest.mark.parametrize("m", [64, 128, 256])
def test_bf16_causal_ragged(n, m):
    cfg = fi.Config("crag", 1, 2, n, 64, m, "bf16", True, 64, "iid", 200 + n)
    x = fi.make_inputs(cfg)
    y = run(x, torch.bfloat16, causal=True)
    assert np.all(np.isfinite(y))
    err = oracle.max_rel_err(y, oracle.attention_causal(x["q"], x["k"], x["v"], x["W"]))
    assert err < TOL_BF16, err


def test_bf16_causal_C2_full_and_entry_points():
    x = fi.make_inputs(fi.config("C2"))
    t = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    y1 = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=True)
    y2 = favor.attention_causal(t["q"], t["k"], t["v"], t["W"], chunk=64)
    y3 = favor.attention_causal(t["q"], t["k"], t["v"], t["W"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    y = y1.cpu().numpy()
    ref = oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])
    err = oracle.max_rel_err(y, ref)
    print(f"C2 causal bf16 err {err:.3e}")
    assert err < TOL_BF16
    # first row is v_0; last row equals the non-causal last row
    assert np.max(np.abs(y[..., 0, :] - x["v"][..., 0, :])) < 2e-3
    ync = run(x, torch.bfloat16)
    assert oracle.max_rel_err(y[..., -1:, :], ync[..., -1:, :]) < TOL_BF16


def _full_causal(cfg_name, **over):
    """The whole causal output at a benchmark shape, every (b, h) slice and row,
    against the oracle's prefix-sum form (slices spread over host processes)."""
    cfg = fi.config(cfg_name, causal=True, **over)
    x = fi.make_inputs(cfg)
    y = run(x, torch.bfloat16, causal=True)
    assert np.all(np.isfinite(y))
    ref = oracle_pool.reference(x, causal=True)
    errs = oracle_pool.slice_errors(y, ref, [(b, h) for b in range(cfg.B) for h in range(cfg.H)])
    worst = max(errs.values())
    print(f"{cfg_name} causal full output: worst slice err {worst:.3e} over {len(errs)} slices")
    return x, y, ref, worst


def test_bf16_causal_C3_shape_full():
    """B=4, H=8, n=16384, m=256 causal: the benchmark's causal call, whole output."""
    _, _, _, worst = _full_causal("C3")
    assert worst < TOL_BF16


def test_bf16_causal_C4_full():
    """B=2, H=12, n=32768, m=256 causal: whole output (segment boundaries included),
    plus the oracle's own check on a 512-token prefix (prefix sums against the
    masked quadratic form)."""
    x, y, ref, worst = _full_causal("C4")
    assert worst < TOL_BF16
    q, k, v, W = x["q"][0, 0, :512], x["k"][0, 0, :512], x["v"][0, 0, :512], x["W"][0]
    quad = oracle.attention_quadratic(q, k, v, W, causal=True)
    assert oracle.max_rel_err(ref[0, 0, :512], quad) < 1e-12


def test_bf16_causal_prefix_consistency_and_determinism():
    cfg = fi.config("C2", H=3, n=3000, causal=True)
    x = fi.make_inputs(cfg)
    t = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    y = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=True)
    y2 = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    half = {k: (v[:, :, :1500].contiguous() if k != "W" else v) for k, v in t.items()}
    yh = favor.attention(half["q"], half["k"], half["v"], half["W"], causal=True)
    torch.cuda.synchronize()
    a = y[:, :, :1500].cpu().numpy()
    b = yh.cpu().numpy()
    assert oracle.max_rel_err(a, b) < 1e-3


@pytest.mark.parametrize("scale", [2.0, 4.0])
def test_bf16_causal_stress(scale):
    cfg = fi.config("C2", H=2, n=2000, causal=True)
    x = fi.make_inputs(cfg, qk_scale=scale)
    y = run(x, torch.bfloat16, causal=True)
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])) < TOL_BF16


@pytest.mark.parametrize("scale", [4.0, 6.0])
def test_bf16_causal_wide_key_spread(scale):
    """The first 8 keys of every 32-key tile have `scale` times the norm, so
    the keys of a diagonal tile differ by far more than 2^32 in their largest
    feature: the chunk term takes per-key shifts there, and rows 0-7 of a
    tile see only the large-norm keys of their own tile."""
    cfg = fi.config("C2", H=2, n=2000, causal=True)
    x = fi.make_inputs(cfg)
    k = x["k"].astype(np.float64)
    sel = (np.arange(k.shape[-2]) % 32) < 8
    k[:, :, sel, :] *= scale
    x["k"] = fi.round_bf16(k)
    y = run(x, torch.bfloat16, causal=True)
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])) < TOL_BF16


def test_bf16_causal_growing_keys():
    """Key norms grow along the sequence, so later chunks raise the running
    per-feature shift many times (the rescale path)."""
    cfg = fi.config("C2", H=2, n=2048, causal=True)
    x = fi.make_inputs(cfg)
    k = x["k"].astype(np.float64)
    k *= np.linspace(0.2, 4.0, k.shape[-2])[None, None, :, None]
    x["k"] = fi.round_bf16(k)
    y = run(x, torch.bfloat16, causal=True)
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])) < TOL_BF16


@pytest.mark.parametrize("limit", [0, 1])
def test_bf16_causal_handover_fallback(limit):
    """The key-tile hand-over's bounded wait, forced short from the host: with
    limit 0 the query tile 1 waves abandon every chunk whose first key tile
    the tile 0 waves have not yet claimed, and compute that tile themselves.
    Every launch completes; each output equals the normal run's bit for bit
    (both ways form the same operands) and meets the oracle's bar."""
    cfg = fi.config("C2", H=4, n=2048, causal=True)
    x = fi.make_inputs(cfg)
    t = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    _lib = favor._lib
    y0 = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=True)
    torch.cuda.synchronize()
    try:
        _lib.check(_lib.favor_set_handover_spin_limit(limit))
        ys = [favor.attention(t["q"], t["k"], t["v"], t["W"], causal=True) for _ in range(3)]
        torch.cuda.synchronize()
    finally:
        _lib.check(_lib.favor_set_handover_spin_limit(4096))
    for y in ys:
        assert torch.equal(y, y0)
    ref = oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])
    assert oracle.max_rel_err(y0.cpu().numpy(), ref) < TOL_BF16


def test_profile_filter_records_one_kernel():
    x = fi.make_inputs(fi.config("C2", H=2, n=512))
    t = {k: dev(v, torch.bfloat16) for k, v in x.items()}
    _lib = favor._lib
    _lib.check(_lib.favor_profile_enable_only("k_output"))
    favor.attention(t["q"], t["k"], t["v"], t["W"])
    torch.cuda.synchronize()
    only = _lib.favor_profile_collect()
    _lib.check(_lib.favor_profile_enable())
    favor.attention(t["q"], t["k"], t["v"], t["W"])
    torch.cuda.synchronize()
    every = _lib.favor_profile_collect()
    assert set(only) == {"k_output"} and only["k_output"][0] == 1
    assert {"k_kv_state", "k_merge", "k_output"} <= set(every)
