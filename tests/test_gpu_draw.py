"""GPU parity of the on-device orthogonal random features against the oracle's
draw (same Philox4x64-10 stream definition, fp64 arithmetic on both sides).

fp32 output: within one fp32 ulp of the oracle's fp64 W.  bf16 output: equal to
the oracle's W rounded once to the nearest bf16 (only a value within ~1e-12 of
a rounding boundary could differ).
"""
import numpy as np
import pytest

import favor_inputs as fi
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import kernelized_linear_attention_favor_amd as favor  # noqa: E402

DEV = torch.device("cuda:0")


def bf16_nearest(x):
    """fp64 -> nearest bf16 (ties to even), rounded once: fp32 rounded to odd
    (truncate, then set the last bit if inexact), then fp32 -> bf16 to nearest."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    inexact = f.astype(np.float64) != x
    over = np.abs(f.astype(np.float64)) > np.abs(x)
    bits = f.view(np.uint32).copy()
    bits[inexact & over] -= 1
    bits[inexact] |= 1
    return fi.round_bf16(bits.view(np.float32))


@pytest.mark.parametrize("H,m,d", [(2, 256, 64), (1, 100, 32), (3, 16, 16), (2, 40, 16), (8, 256, 64)])
def test_draw_matches_oracle(H, m, d):
    seed, step = 1234, 7
    ref = oracle.draw_features(seed, step, H, m, d)
    w32 = favor.draw_features(seed, step, H, m, d, dtype=torch.float32).cpu().numpy()
    r32 = ref.astype(np.float32)
    assert np.all(np.abs(w32.astype(np.float64) - r32) <= np.spacing(np.abs(r32)))
    wbf = favor.draw_features(seed, step, H, m, d).float().cpu().numpy()
    assert np.array_equal(wbf, bf16_nearest(ref))


def test_draw_is_deterministic_and_redraws():
    a = favor.draw_features(5, 0, 4, 128, 64, dtype=torch.float32)
    b = favor.draw_features(5, 0, 4, 128, 64, dtype=torch.float32)
    c = favor.draw_features(5, 1, 4, 128, 64, dtype=torch.float32)
    d = favor.draw_features(6, 0, 4, 128, 64, dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert (a - c).abs().max().item() > 0.5 and (a - d).abs().max().item() > 0.5
    # large seeds and steps (all 64 bits) match the oracle too
    big = (2**64 - 3, 2**63 + 11)
    w = favor.draw_features(*big, 1, 64, 64, dtype=torch.float32).cpu().numpy()
    r = oracle.draw_features(*big, 1, 64, 64).astype(np.float32)
    assert np.all(np.abs(w.astype(np.float64) - r) <= np.spacing(np.abs(r)))


def test_drawn_blocks_are_orthogonal():
    W = favor.draw_features(9, 3, 2, 256, 64, dtype=torch.float32).double().cpu().numpy()
    for h in range(2):
        for b in range(4):
            Wb = W[h, 64 * b:64 * b + 64]
            G = Wb @ Wb.T
            s2 = np.diag(G)
            assert np.all(s2 > 0)
            off = G - np.diag(s2)
            assert np.max(np.abs(off)) < 1e-5 * np.max(s2)


def test_attention_with_drawn_features():
    """The path fed by the device draw: FAVOR+ attention with the drawn bf16 W
    against the oracle with the oracle's draw (rounded the same way)."""
    cfg = fi.config("C2")
    x = fi.make_inputs(cfg)
    Wg = favor.draw_features(77, 0, cfg.H, cfg.m, cfg.d)
    Wr = bf16_nearest(oracle.draw_features(77, 0, cfg.H, cfg.m, cfg.d))
    t = {k: torch.from_numpy(v).to(DEV, torch.bfloat16) for k, v in x.items() if k != "W"}
    for causal in (False, True):
        y = favor.attention(t["q"], t["k"], t["v"], Wg, causal=causal).cpu().numpy()
        f = oracle.attention_causal if causal else oracle.attention
        assert oracle.max_rel_err(y, f(x["q"], x["k"], x["v"], Wr)) < 2e-3


def test_bf16_nearest_reference_rounds_once():
    # the tie that two roundings get wrong: just below the bf16 midpoint of
    # 1.2421875 and 1.25, whose fp32 rounding is the midpoint itself
    x = np.array([1.2460937449402247, 1.24609375, 1.2460937550597753, -1.2460937449402247])
    assert list(bf16_nearest(x)) == [1.2421875, 1.25, 1.25, -1.2421875]
