"""Host-side logic of bench.py (CPU only): the algorithmic byte counts the
roofline divides by, the percentile summary, the sources digest that ties the
committed HBM-traffic counters to the kernel sources, and the one-GPU guard."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("favor_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes(bench):
    # per (b, h): q, k, v read once as bf16 (2 B), y written once as fp32 (4 B);
    # W (bf16 [H, m, d]) read once per launch
    B, H, n, d, m = 4, 8, 16384, 64, 256
    tok = B * H * n * d
    W = H * m * d * 2
    assert bench.kernel_bytes("k_causal_output", B, H, n, d, m) == 3 * tok * 2 + tok * 4 + W == 335806464
    assert bench.kernel_bytes("k_kv_state", B, H, n, d, m) == 2 * tok * 2 + W == 134479872
    assert bench.kernel_bytes("k_output", B, H, n, d, m) == tok * 2 + tok * 4 + W == 201588736
    # one causal call: 10 n d bytes per (b, h) (three bf16 inputs, one fp32 output) plus W
    assert bench.kernel_bytes("k_causal_output", B, H, n, d, m) == 10 * B * H * n * d + W
    assert bench.kernel_bytes("no_such_kernel", B, H, n, d, m) == 0.0


def test_percentiles(bench):
    xs = [float(v) for v in range(1, 12)]   # 1 .. 11
    d = bench.dist(list(reversed(xs)))
    assert d["median_us"] == 6.0 and d["p10_us"] == 2.0 and d["p90_us"] == 10.0
    assert d["mean_us"] == 6.0 and d["calls"] == 11
    # linear interpolation between order statistics
    assert bench._pct([0.0, 10.0], 0.25) == 2.5
    assert bench._pct([], 0.5) is None


def test_digest_ignores_comments(bench):
    a = "int f(int x) {\n  return x + 1;  // one\n}\n"
    b = "/* header\n   comment */\nint f(int x) {\n\n  return x + 1;\n}   \n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("+ 1", "+ 2"))
    d = bench.source_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    assert bench.source_digest() == d   # stable


def test_traffic_lookup(bench):
    assert bench.read_traffic("k_causal_output", "0" * 16) is None
    d = bench.source_digest()
    t = bench.read_traffic("k_causal_output", d)
    if t is None:
        pytest.skip("the committed counters were taken on other kernel sources")
    # HBM bytes counted for the chunk kernel cover at least what it must move
    assert t >= bench.kernel_bytes("k_causal_output", 4, 8, 16384, 64, 256)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
