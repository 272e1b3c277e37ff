"""Checks of the seeded input generators (random W structure, bf16 rounding, shapes)."""
import math

import numpy as np
import pytest
from scipy import stats

import favor_inputs as fi


def test_orthogonal_blocks_and_norms():
    rng = np.random.default_rng(1)
    H, m, d = 3, 40, 16                      # 2 full blocks + a truncated third
    W = fi.orthogonal_W(rng, H, m, d)
    assert W.shape == (H, m, d)
    for h in range(H):
        for b0 in range(0, m, d):
            Wb = W[h, b0:b0 + d]
            G = Wb @ Wb.T
            s2 = np.sum(Wb * Wb, axis=1)
            assert np.max(np.abs(G - np.diag(s2))) < 1e-12 * np.max(s2)


def test_row_norms_are_chi_d():
    rng = np.random.default_rng(2)
    d = 16
    W = fi.orthogonal_W(rng, 200, 32, d)
    norms = np.linalg.norm(W, axis=-1).ravel()
    p = stats.kstest(norms, stats.chi(d).cdf).pvalue
    assert p > 1e-3


def test_entries_standard_normal_marginal():
    rng = np.random.default_rng(3)
    W = fi.orthogonal_W(rng, 100, 64, 16)
    e = W.ravel()
    assert abs(e.mean()) < 0.02
    assert abs(e.var() - 1) < 0.03
    p = stats.kstest(W[:, 5, 3], "norm").pvalue
    assert p > 1e-3


def test_round_bf16_rne_and_exactness():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0, 3.0e38, np.inf, -np.inf])
    r = fi.round_bf16(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to even (1.0)
    assert r[0] == 1.0 and r[1] == 1.0
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6: even mantissa is 1 + 2^-6
    assert r[2] == 1.0 + 2 ** -6
    assert r[3] == 1.0
    assert r[4] == -2.5 and r[5] == 0.0
    assert np.isinf(r[7]) and np.isinf(r[8])
    rng = np.random.default_rng(4)
    y = rng.standard_normal(10000) * 10
    ry = fi.round_bf16(y)
    assert np.all(np.abs(ry - y) <= np.abs(y) * 2 ** -8 * 1.0001)
    assert np.array_equal(fi.round_bf16(ry), ry)
    assert np.array_equal(fi.bits_to_f32(fi.bf16_bits(ry)), ry)
    assert np.isnan(fi.round_bf16(np.array([np.nan]))[0])


def test_round_bf16_against_torch():
    import torch
    rng = np.random.default_rng(5)
    y = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    want = torch.from_numpy(y).to(torch.bfloat16).float().numpy()
    assert np.array_equal(fi.round_bf16(y), want)


@pytest.mark.parametrize("name", ["C1", "C2", "C5"])
def test_make_inputs_shapes_and_determinism(name):
    cfg = fi.config(name)
    if cfg.B * cfg.H * cfg.n > 200000:
        cfg = cfg.replace(B=1, H=2)
    a = fi.make_inputs(cfg)
    b = fi.make_inputs(cfg)
    for key in ("q", "k", "v", "W"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == cfg.shape and a["W"].shape == (cfg.H, cfg.m, cfg.d)
    if cfg.dtype == "bf16":
        for key in ("q", "k", "v", "W"):
            assert np.array_equal(fi.round_bf16(a[key]), a[key])
    c = fi.make_inputs(cfg, set_index=1)
    assert not np.array_equal(a["q"], c["q"])
    # Q, K scaled by d^-1/4: mean |q|^2 is about sqrt(d)
    qn = np.mean(np.sum(a["q"].astype(np.float64) ** 2, axis=-1))
    assert abs(qn / math.sqrt(cfg.d) - 1) < 0.1


def test_configs_match_workloads():
    c = fi.CONFIGS
    assert (c["C1"].B, c["C1"].H, c["C1"].n, c["C1"].d, c["C1"].m, c["C1"].dtype) == (1, 1, 256, 32, 64, "f32")
    assert (c["C2"].B, c["C2"].H, c["C2"].n, c["C2"].d, c["C2"].m) == (1, 8, 1024, 64, 256)
    assert (c["C3"].B, c["C3"].H, c["C3"].n, c["C3"].d, c["C3"].m) == (4, 8, 16384, 64, 256)
    assert (c["C4"].B, c["C4"].H, c["C4"].n, c["C4"].d, c["C4"].m, c["C4"].causal, c["C4"].chunk) == (2, 12, 32768, 64, 256, True, 64)
    assert (c["C5"].B, c["C5"].H, c["C5"].n, c["C5"].d, c["C5"].m, c["C5"].qk) == (32, 12, 4096, 64, 128, "lowrank")
