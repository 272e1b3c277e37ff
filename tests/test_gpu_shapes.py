"""GPU parity of the bf16 path over its whole shape range, against the fp64 oracle.

The shape range: head dimension d in {32, 64}; feature count m any multiple of
16 from 16 to 512 (features run in 32-feature tiles, the tail of the last tile
masked; more than 256 features, or 128 with chunks of 128, are cut into slices
whose partials a final kernel combines); causal chunk length in {16, 32, 64,
128}.  Sequence lengths are ragged (n = 1, 31, 65, 4097), so the last tile,
chunk and key range are partial.  Bar: max over (b, h) of max|y - y_ref| /
max|y_ref| <= 2e-3 (the bf16 bar).
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
NS = [1, 31, 65, 4097]


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=torch.bfloat16)


def inputs(B, H, n, d, m, seed):
    return fi.make_inputs(fi.Config("shape", B, H, n, d, m, "bf16", False, 64, "iid", seed))


def gpu(x, causal, chunk=0):
    t = {k: bf(v) for k, v in x.items()}
    if causal and chunk:
        y = favor.attention_causal(t["q"], t["k"], t["v"], t["W"], chunk=chunk)
    else:
        y = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=causal)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(x, y, causal):
    assert np.all(np.isfinite(y))
    B, H = x["q"].shape[:2]
    if B * H >= 8:
        ref = oracle_pool.reference(x, causal=causal)   # one (b, h) slice per host process
    else:
        ref = (oracle.attention_causal if causal else oracle.attention)(x["q"], x["k"], x["v"], x["W"])
    err = oracle.max_rel_err(y, ref)
    assert err < TOL, err
    return err


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("m", [16, 48, 96, 192, 288, 320, 512])
@pytest.mark.parametrize("n", NS)
def test_feature_counts(n, m, causal):
    """m in 16Z beyond {64, 128, 256}: a masked half tile (16, 48), odd tile counts
    (96, 192: 3 and 6 waves), the largest table two output workgroups share a CU
    with (288), and feature slices in the causal walk (288, 320, 512)."""
    x = inputs(1, 2, n, 64, m, 1000 + m + n)
    check(x, gpu(x, causal), causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("m", [32, 64, 256, 512])
@pytest.mark.parametrize("n", NS)
def test_head_dim_32(n, m, causal):
    x = inputs(1, 2, n, 32, m, 2000 + m + n)
    check(x, gpu(x, causal), causal)


@pytest.mark.parametrize("m", [64, 256, 320])
@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
@pytest.mark.parametrize("n", NS)
def test_chunk_lengths(n, chunk, m):
    """The causal walk with every chunk length (m = 320 with chunks of 128 runs
    three slices in two launch groups)."""
    x = inputs(1, 2, n, 64, m, 3000 + chunk + m + n)
    check(x, gpu(x, True, chunk), True)


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
@pytest.mark.parametrize("m", [64, 256])
def test_long_walks(m, chunk, d):
    """Many (b, h) pairs, so that each segment is walked over many chunks (about
    500 tokens per segment), with the carry from the earlier segments."""
    x = inputs(2, 16, 4097, d, m, 4000 + chunk + m + d)
    check(x, gpu(x, True, chunk), True)


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
@pytest.mark.parametrize("scale", [2.0, 4.0])
def test_chunk_lengths_stress(chunk, scale):
    """Q, K scaled up (exponent spreads beyond the fast path's limit in many
    chunks): every chunk length stays finite and within the bar."""
    cfg = fi.config("C2", H=2, n=2000, causal=True)
    x = fi.make_inputs(cfg, qk_scale=scale)
    check(x, gpu(x, True, chunk), True)


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_chunk_lengths_wide_key_spread(chunk):
    """The first 8 keys of every 32 have 6 times the norm: chunks whose keys
    spread far below their features' shifts take the per-row slow path."""
    cfg = fi.config("C2", H=2, n=1500, causal=True)
    x = fi.make_inputs(cfg)
    k = x["k"].astype(np.float64)
    k[:, :, (np.arange(k.shape[-2]) % 32) < 8, :] *= 6.0
    x["k"] = fi.round_bf16(k)
    check(x, gpu(x, True, chunk), True)


def test_chunk_lengths_agree():
    """The chunk length is how the prefix sums are cut, not what they are: all
    four give the oracle's result, and each other's within twice the bar."""
    x = inputs(1, 4, 3000, 64, 256, 5000)
    ys = [gpu(x, True, c) for c in (16, 32, 64, 128)]
    ref = oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])
    for y in ys:
        assert oracle.max_rel_err(y, ref) < TOL
    for y in ys[1:]:
        assert oracle.max_rel_err(y, ys[0]) < 2 * TOL


def test_d32_matches_zero_padded_d64():
    """A d = 32 call equals the d = 64 call on the same inputs padded with zero
    columns (|x|^2 and w.x are unchanged; the extra value columns are 0), up to
    rounding: both within the bar of the oracle and of each other."""
    x = inputs(1, 2, 1500, 32, 128, 6000)
    pad = {k: np.concatenate([v, np.zeros(v.shape[:-1] + (32,), np.float32)], axis=-1) for k, v in x.items()}
    for causal in (False, True):
        y32 = gpu(x, causal)
        y64 = gpu(pad, causal)
        assert np.max(np.abs(y64[..., 32:])) == 0.0
        assert oracle.max_rel_err(y32, y64[..., :32]) < TOL


def test_walk_benchmark_shape_chunk32_full():
    """B=4, H=8, n=16384, m=256 causal with chunks of 32 (the general walk at the
    benchmark shape; chunks of 64 there take the specialised kernel): the whole
    output against the oracle."""
    x = fi.make_inputs(fi.config("C3", causal=True))
    y = gpu(x, True, 32)
    assert np.all(np.isfinite(y))
    ref = oracle_pool.reference(x, causal=True)
    errs = oracle_pool.slice_errors(y, ref, [(b, h) for b in range(4) for h in range(8)])
    assert max(errs.values()) < TOL, max(errs.values())
