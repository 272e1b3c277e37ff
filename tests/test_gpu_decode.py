"""GPU parity of the streaming decode path (state reset, state of a key
sequence, token-by-token decode) against the fp64 oracle.

Decode runs in fp32 from bf16 inputs, so its bar is the fp32 one (1e-5, per
(b,h) max|y - y_ref| / max|y_ref|); a state built by favor_state_from_keys
goes through the bf16 state kernels (fp16 key features), so outputs that
depend on it meet the bf16 bar (2e-3).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import favor_inputs as fi
import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU, skipped by the marker
    pytest.skip("no GPU", allow_module_level=True)

import kernelized_linear_attention_favor_amd as favor  # noqa: E402

TOL_F32 = 1e-5
TOL_BF16 = 2e-3
dev = torch.device("cuda:0")


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=torch.bfloat16)


def decode_in_calls(x, sizes, state):
    """Decode the tokens of x in consecutive calls of the given sizes."""
    ys, s0 = [], 0
    for T in sizes:
        sl = slice(s0, s0 + T)
        ys.append(favor.decode(bf(x["q"][..., sl, :]), bf(x["k"][..., sl, :]), bf(x["v"][..., sl, :]),
                               bf(x["W"]), state))
        s0 += T
    torch.cuda.synchronize()
    return torch.cat(ys, dim=2).cpu().numpy()


def plain_state(state):
    """The oracle's S = Phi(K)^T V and z = Phi(K)^T 1 from a library state: the
    state carries 2^-c_f per feature and leaves out phi's 1/sqrt(m)."""
    S, z, c = (t.cpu().numpy().astype(np.float64) for t in state.tensors())
    sc = np.exp2(c) / np.sqrt(state.m)
    return S * sc[..., None], z * sc


@pytest.mark.parametrize("m", [64, 128, 256])
@pytest.mark.parametrize("sizes", [[1] * 20, [7, 1, 64, 28]])
def test_decode_from_empty_matches_oracle(m, sizes):
    n = sum(sizes)
    cfg = fi.Config("dec", 1, 3, n, 64, m, "bf16", True, 64, "iid", 700 + m + n)
    x = fi.make_inputs(cfg)
    st = favor.State(1, 3, 64, m)
    y = decode_in_calls(x, sizes, st)
    yref, Sref, zref = oracle.decode(x["q"], x["k"], x["v"], x["W"])
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, yref) < TOL_F32
    assert oracle.max_rel_err(y, oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])) < TOL_F32
    S, z = plain_state(st)
    assert oracle.max_rel_err(S, Sref) < TOL_F32
    np.testing.assert_allclose(z, zref, rtol=TOL_F32)


@pytest.mark.parametrize("B,H", [(2, 128), (4, 128), (8, 128)])
def test_decode_wide_column_slices(B, H):
    """Grids of many heads give each workgroup a wider column slice (16, 32 and
    64 value columns for 256, 512 and 1024 heads); 37 tokens cross a 32-token
    block inside one call."""
    cfg = fi.Config("dec", B, H, 37, 64, 64, "bf16", True, 64, "iid", 800 + B)
    x = fi.make_inputs(cfg)
    st = favor.State(B, H, 64, 64)
    y = decode_in_calls(x, [3, 34], st)
    yref, Sref, zref = oracle.decode(x["q"], x["k"], x["v"], x["W"])
    assert oracle.max_rel_err(y, yref) < TOL_F32
    S, z = plain_state(st)
    assert oracle.max_rel_err(S, Sref) < TOL_F32
    np.testing.assert_allclose(z, zref, rtol=TOL_F32)


def test_decode_splits_are_bitwise_identical():
    cfg = fi.Config("dec", 2, 2, 96, 64, 256, "bf16", True, 64, "iid", 731)
    x = fi.make_inputs(cfg)
    a = decode_in_calls(x, [96], favor.State(2, 2, 64, 256))
    b = decode_in_calls(x, [1] * 96, favor.State(2, 2, 64, 256))
    c = decode_in_calls(x, [13, 50, 33], favor.State(2, 2, 64, 256))
    assert np.array_equal(a, b) and np.array_equal(a, c)
    assert np.max(np.abs(a[..., 0, :] - x["v"][..., 0, :])) < 1e-6   # y_0 = v_0


@pytest.mark.parametrize("scale", [2.0, 4.0])
def test_decode_large_logits(scale):
    cfg = fi.config("C2", H=2, n=300, causal=True)
    x = fi.make_inputs(cfg, qk_scale=scale)
    y = decode_in_calls(x, [300], favor.State(1, 2, 64, cfg.m))
    assert np.all(np.isfinite(y))
    assert oracle.max_rel_err(y, oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])) < TOL_F32


@pytest.mark.parametrize("m,n", [(64, 1), (128, 65), (256, 1000)])
def test_state_from_keys_then_decode(m, n):
    T = 40
    cfg = fi.Config("dec", 1, 2, n + T, 64, m, "bf16", True, 64, "iid", 750 + n)
    x = fi.make_inputs(cfg)
    st = favor.State(1, 2, 64, m)
    st.buf.fill_(7.0)   # from_keys replaces every word, the finish counters included
    st.from_keys(bf(x["k"][..., :n, :]), bf(x["v"][..., :n, :]), bf(x["W"]))
    torch.cuda.synchronize()
    Sref, zref = oracle.kv_state(x["k"][..., :n, :], x["v"][..., :n, :], x["W"])
    S, z = plain_state(st)
    # the state's own rounding: fp16 key features, so the bf16 bar (S relative
    # to its largest entry per (b,h); z relative per feature)
    assert oracle.max_rel_err(S, Sref) < TOL_BF16
    np.testing.assert_allclose(z, zref, rtol=TOL_BF16)
    y = decode_in_calls({k: v[..., n:, :] if k != "W" else v for k, v in x.items()}, [T], st)
    ref = oracle.attention_causal(x["q"], x["k"], x["v"], x["W"])[..., n:, :]
    assert oracle.max_rel_err(y, ref) < TOL_BF16


def test_reset_clears_the_state():
    cfg = fi.Config("dec", 1, 2, 30, 64, 128, "bf16", True, 64, "iid", 777)
    x = fi.make_inputs(cfg)
    st = favor.State(1, 2, 64, 128)
    a = decode_in_calls(x, [30], st)
    st.reset()
    b = decode_in_calls(x, [30], st)
    assert np.array_equal(a, b)
    S, z, c = st.tensors()
    st.reset()
    torch.cuda.synchronize()
    assert torch.all(S == 0) and torch.all(z == 0) and torch.all(torch.isneginf(c))


def test_decode_after_C3_prompt_sampled():
    """A C3-shaped prompt (B=4, H=8, n=16384, m=256) into the state, then 64
    decoded tokens; the oracle checks two (b,h) slices."""
    cfg = fi.config("C3")
    T = 64
    x = fi.make_inputs(cfg)
    rng = np.random.default_rng(99)
    xt = {k: (rng.standard_normal(x["q"].shape[:2] + (T, 64)) * (64 ** -0.25 if k != "v" else 1.0))
          for k in ("q", "k", "v")}
    xt = {k: fi.round_bf16(v) for k, v in xt.items()}
    st = favor.State(cfg.B, cfg.H, 64, cfg.m)
    st.from_keys(bf(x["k"]), bf(x["v"]), bf(x["W"]))
    y = decode_in_calls({**xt, "W": x["W"]}, [T], st)
    for b, h in ((0, 0), (3, 7)):
        S0, z0 = oracle.kv_state(x["k"][b, h], x["v"][b, h], x["W"][h])
        yref, _, _ = oracle.decode(xt["q"][b, h], xt["k"][b, h], xt["v"][b, h], x["W"][h], S0, z0)
        assert oracle.max_rel_err(y[b, h], yref) < TOL_BF16
