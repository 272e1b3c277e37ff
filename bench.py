#!/usr/bin/env python3
"""Benchmark of the FAVOR+ attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
non-causal FAVOR+ attention (feature map, key/value state, output) followed by
causal FAVOR+ attention (chunked prefix sums) on the same batch.  Workload:
B=4, H=8, n=16384, d=64, m=256, bf16 inputs, fp32 outputs.  Several
independent input sets rotate between steps so that the 256 MB Infinity Cache
cannot hold a step's working set.  Inputs are resident in HBM before timing.

Prints one JSON line:
  value          tokens/s for the step (B*n tokens per step); the timed region
                 holds the K steps only, with events at its two ends
  roofline       dominant kernel: algorithmic bytes per launch / mean launch
                 time (HIP events around that kernel alone, on its launch
                 stream, in a separate pass), against 8 TB/s HBM
  cpu_baseline   the fp64 oracle timed on host cores on a sample of the same
                 workload (whole (b, h) slices)
  per_call       per-call kernel totals and median / p10 / p90 call times
  valu, rates    instruction-rate probes (v_exp_f32, v_fma_f32) and each
                 exp-forming kernel's exponential floor at the measured rate
  workloads      the causal n=32768 and vision-style workloads, per call
  environment    GPU, clocks, ROCm / HIP versions, the library file timed
and, each measured outside the timed step with its own HIP events and the
oracle timed beside it: decode (streaming decode on the same shape),
feature_maps (ReLU and elu+1 maps), feature_draw (on-device W), backward and
backward_causal (dq, dk, dv for an upstream gradient).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
FP64_PEAK_TFLOPS = 78.6         # MI355X fp64 vector, published
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
CSRC = os.path.join(ROOT, "kernelized_linear_attention_favor_amd", "csrc")


def kernel_bytes(name: str, B: int, H: int, n: int, d: int, m: int) -> float:
    """Algorithmic HBM bytes one launch of `name` must move (inputs read once,
    outputs written once; bf16 inputs, fp32 outputs)."""
    BH = B * H
    tok = BH * n * d
    W = H * m * d * 2
    table = {
        "k_kv_state": 2 * tok * 2 + W,               # K, V
        "k_output": tok * 2 + tok * 4 + W,           # Q in, y out
        "k_causal_state": 2 * tok * 2 + W,           # K, V
        "k_causal_output": 3 * tok * 2 + tok * 4 + W,  # Q, K, V in, y out
        "k_causal_walk": 3 * tok * 2 + tok * 4 + W,    # Q, K, V in, y out (the general causal walk)
        # backward: bf16 q, k, v and fp32 y, dy, aux (M, D, delta) in; fp32 dq, dk, dv out
        "k_bw_query": tok * 2 + 2 * tok * 4 + tok * 4 + BH * n * 16 + W,         # q, y, dy -> dq, aux
        "k_bw_key": 2 * tok * 2 + 2 * tok * 4 + W,                              # k, v -> dk, dv
        "k_bw_query_causal": 3 * tok * 2 + 2 * tok * 4 + tok * 4 + BH * n * 16 + W,
        "k_bw_key_causal": 3 * tok * 2 + tok * 4 + BH * n * 16 + 2 * tok * 4 + W,  # q, k, v, dy, aux -> dk, dv
    }
    return float(table.get(name, 0.0))


def _code_only(text: str) -> str:
    """Source text without comments, trailing blanks and empty lines (the
    device sources hold no "//" inside string literals)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (ln.split("//", 1)[0].rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln.strip())


def source_digest() -> str:
    """Digest of the device code (kernels and their headers, comments left out;
    the host layer does not change what the counters measure)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith((".hip", ".h")):
            continue
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(f.encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, digest: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources; else None."""
    if not os.path.exists(PMC_FILE):
        return None
    for line in open(PMC_FILE):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kv = dict(tok.split("=", 1) for tok in line.split() if "=" in tok)
        if kv.get("kernel") == kernel and kv.get("sources") == digest and "bytes_per_launch" in kv:
            return float(kv["bytes_per_launch"])
    return None


def _pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    k = (len(xs) - 1) * q
    lo = int(k)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def dist(us_list) -> dict:
    """median / p10 / p90 / mean of a list of per-call times (microseconds)."""
    return {"median_us": round(_pct(us_list, 0.5), 2), "p10_us": round(_pct(us_list, 0.1), 2),
            "p90_us": round(_pct(us_list, 0.9), 2), "mean_us": round(sum(us_list) / len(us_list), 2),
            "calls": len(us_list)}


def dpm_clocks(props):
    """Current shader and memory clock levels of the device, read from the
    driver's sysfs DPM tables (the level marked '*').  Read in-process: a tool
    started as a child would inherit a profiler's preload.  None if the tables
    are not visible."""
    import glob
    want = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}"
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            if not os.path.basename(os.path.realpath(dev)).startswith(want):
                continue
            out = []
            for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
                with open(os.path.join(dev, name)) as fh:
                    cur = [ln.strip() for ln in fh if ln.rstrip().endswith("*")]
                out.append(f"{name[7:]} {cur[0].rstrip(' *')}" if cur else f"{name[7:]} ?")
            return out
        except OSError:
            continue
    return None


def environment(torch) -> dict:
    """GPU, clocks, software versions and the library that was timed."""
    props = torch.cuda.get_device_properties(0)
    env = {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count, "hip": torch.version.hip, "torch": torch.__version__}
    try:
        with open("/opt/rocm/.info/version") as fh:
            env["rocm"] = fh.read().strip()
    except OSError:
        env["rocm"] = None
    env["clocks"] = dpm_clocks(props)
    from kernelized_linear_attention_favor_amd import _lib as L
    h = hashlib.sha256()
    with open(L.LIB_PATH, "rb") as fh:
        h.update(fh.read())
    env["library"] = {"path": os.path.relpath(L.LIB_PATH, ROOT), "sha256": h.hexdigest()[:16]}
    return env


def probe_rates(torch) -> dict | None:
    """Vector-unit rates from libfavor_ubench (v_exp_f32, v_fma_f32, both
    interleaved), per second over the whole chip.  None if the probe library
    is missing."""
    import ctypes
    path = os.path.join(ROOT, "kernelized_linear_attention_favor_amd", "libfavor_ubench.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    blocks, threads, iters = 8192, 256, 2048
    out = torch.empty(blocks * threads, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    res = {}
    for name, per_iter in (("exp2", (8, 0)), ("fma", (0, 8)), ("mix", (8, 32))):
        fn = getattr(L, f"favor_ubench_{name}")
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        assert fn(out.data_ptr(), blocks, threads, 16, st) == 0
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert fn(out.data_ptr(), blocks, threads, iters, st) == 0
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        t = sorted(times)[len(times) // 2]
        lanes = blocks * threads * iters
        res[name] = {"exp_per_s": lanes * per_iter[0] / t, "fma_per_s": lanes * per_iter[1] / t,
                     "seconds": t}
    return {
        "exp2_per_s": round(res["exp2"]["exp_per_s"], -9),
        "fma_per_s": round(res["fma"]["fma_per_s"], -9),
        "mix_exp_per_s": round(res["mix"]["exp_per_s"], -9),
        "mix_fma_per_s": round(res["mix"]["fma_per_s"], -9),
        "note": "lane operations per second over the chip; mix interleaves 1 exp with 4 fma per chain step",
    }


def exps_per_launch(name: str, B: int, H: int, n: int, m: int) -> float:
    """Exponentials a kernel must evaluate per launch: one per (token, feature)
    pair on each side it forms features for (the causal chunk kernel forms the
    query features, the key features of the running state and the key features
    of the chunk term)."""
    tf = float(B * H * n * m)
    return {"k_kv_state": tf, "k_causal_state": tf, "k_output": tf, "k_causal_output": 3 * tf,
            "k_causal_walk": 2 * tf}.get(name, 0.0)


# ----------------------------------------------------------- CPU baseline
_ORACLE_INPUT = None


def _oracle_slice(args):
    b, h, causal = args
    import oracle  # cpu_baseline leg only
    q, k, v, W = (_ORACLE_INPUT[key] for key in ("q", "k", "v", "W"))
    f = oracle.attention_causal if causal else oracle.attention
    f(q[b, h], k[b, h], v[b, h], W[h])
    return 1


def cpu_baseline(x, cfg, with_causal: bool, budget_s: float = 10.0) -> dict:
    """Time the fp64 oracle (as it stands) on whole (b, h) slices of the workload."""
    global _ORACLE_INPUT
    _ORACLE_INPUT = x
    host = len(os.sched_getaffinity(0))
    cores = min(host, 16)   # a GPU machine's CPU share is 16 cores for one GPU, whatever it reports
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    slices = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    done = 0
    with ctx.Pool(cores) as pool:
        # one round of `cores` slices, repeated until the time budget is used
        i = 0
        while True:
            batch = [slices[(i + j) % len(slices)] for j in range(cores)]
            i += cores
            jobs = [(b, h, False) for b, h in batch]
            if with_causal:
                jobs += [(b, h, True) for b, h in batch]
            sum(pool.map(_oracle_slice, jobs, chunksize=1))
            done += len(batch)
            if time.perf_counter() - t0 >= budget_s or done >= 4 * len(slices):
                break
    wall = time.perf_counter() - t0
    tokens = done / cfg.H * cfg.n   # a token = one query position through all H heads
    variants = "non-causal + causal" if with_causal else "non-causal"
    return {
        "value": tokens / wall,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} whole (b,h) slices of n={cfg.n} (d={cfg.d}, m={cfg.m}) through {variants} "
                  f"fp64 NumPy oracle in {wall:.1f} s on {cores} worker processes (one per core; "
                  f"{host} cores visible, capped at 16, the CPU share of one GPU)",
        "host_cores_visible": host,
        "cpu_model": _cpu_model(),
    }


def _cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------- streaming decode
def decode_bytes(B: int, H: int, T: int, d: int, m: int) -> float:
    """Algorithmic HBM bytes of one decode call: the fp32 state (S, z, c) read
    and written once, W read once, T tokens of bf16 q, k, v in, fp32 y out."""
    state = 4.0 * B * H * m * (d + 2)
    return 2 * state + 2.0 * H * m * d + 3 * 2.0 * B * H * T * d + 4.0 * B * H * T * d


def bench_decode(favor, _lib, torch, fi, cfg, t0, dev, calls: int = 256, t_long: int = 64,
                 cpu_budget_s: float = 2.0) -> dict:
    """Streaming decode on the workload's shape: the prompt (n keys of input set
    0) into a state, then `calls` single-token calls and a few `t_long`-token
    calls.  Kernel times from HIP events around each launch on its stream."""
    B, H, n, d, m = cfg.B, cfg.H, cfg.n, cfg.d, cfg.m
    W = t0["W"]
    st = favor.State(B, H, d, m)
    gen = torch.Generator(device="cpu").manual_seed(4242)

    def toks(T):
        s = (d ** -0.25)
        return [(torch.randn((B, H, T, d), generator=gen) * sc).to(device=dev, dtype=torch.bfloat16)
                for sc in (s, s, 1.0)]

    one = [toks(1) for _ in range(calls)]
    many = [toks(t_long) for _ in range(4)]
    out1 = torch.empty((B, H, 1, d), dtype=torch.float32, device=dev)
    outT = torch.empty((B, H, t_long, d), dtype=torch.float32, device=dev)

    def prompt():
        st.from_keys(t0["k"], t0["v"], W)

    # warm every kernel once
    prompt()
    favor.decode(*one[0], W, st, out=out1)
    favor.decode(*many[0], W, st, out=outT)
    torch.cuda.synchronize()

    _lib.check(_lib.favor_profile_enable())
    for _ in range(3):
        prompt()
    torch.cuda.synchronize()
    pp = _lib.favor_profile_collect()
    prompt_us = sum(t / c for c, t in pp.values()) * 1e3

    prompt()
    _lib.check(_lib.favor_profile_enable_only("k_decode"))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for q, k, v in one:
        favor.decode(q, k, v, W, st, out=out1)
    e1.record()
    torch.cuda.synchronize()
    c1, tt1 = _lib.favor_profile_collect()["k_decode"]
    us1 = tt1 / c1 * 1e3
    wall1 = e0.elapsed_time(e1) / calls * 1e3

    _lib.check(_lib.favor_profile_enable_only("k_decode"))
    for q, k, v in many:
        favor.decode(q, k, v, W, st, out=outT)
    torch.cuda.synchronize()
    cT, ttT = _lib.favor_profile_collect()["k_decode"]
    usT = ttT / cT * 1e3
    assert bool(torch.isfinite(outT).all()), "decode produced non-finite outputs"

    b1 = decode_bytes(B, H, 1, d, m)
    bT = decode_bytes(B, H, t_long, d, m)

    # the oracle's recurrence, timed on a few whole (b, h) slices
    import oracle  # cpu_baseline leg only
    xs = {k: v.float().cpu().numpy() for k, v in zip("qkv", many[0])}
    Wh = W.float().cpu().numpy()
    slices, tc = 0, time.perf_counter()
    while True:
        b, h = divmod(slices % (B * H), H)
        oracle.decode(xs["q"][b, h], xs["k"][b, h], xs["v"][b, h], Wh[h])
        slices += 1
        if time.perf_counter() - tc >= cpu_budget_s:
            break
    cpu_wall = time.perf_counter() - tc
    return {
        "workload": f"prompt n={n} into the state, then decode B={B} H={H} d={d} m={m}",
        "state_bytes": int(_lib.favor_state_bytes(B, H, d, m)),
        "prompt_to_state_us": round(prompt_us, 2),
        "T1": {"kernel_us": round(us1, 2), "wall_us_per_call": round(wall1, 2),
               "tokens_per_s": round(B / (us1 * 1e-6), 1), "bytes_per_launch": b1,
               "hbm_frac": round(b1 / (us1 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        f"T{t_long}": {"kernel_us": round(usT, 2), "tokens_per_s": round(B * t_long / (usT * 1e-6), 1),
                       "bytes_per_launch": bT,
                       "hbm_frac": round(bT / (usT * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "cpu_baseline": {"value": round(slices * t_long / H / cpu_wall, 1), "unit": "tokens/s", "cores": 1,
                         "kind": "oracle",
                         "sample": f"{slices} (b,h) slices of {t_long} tokens through the fp64 oracle's "
                                   f"decode recurrence in {cpu_wall:.1f} s, one process"},
    }


# ---------------------------------------------------- deterministic feature maps
def bench_phi(favor, _lib, torch, cfg, sets, dev, steps: int, cpu_budget_s: float) -> dict:
    """The ReLU (m = 256) and elu(x)+1 (m = d) feature maps on the workload's
    shape: non-causal and causal calls, per-kernel HIP-event times, and the
    oracle timed on whole (b, h) slices beside them."""
    B, H, n, d = cfg.B, cfg.H, cfg.n, cfg.d
    res = {}
    for kind, m in (("relu", cfg.m), ("elu1", d)):
        W = sets[0]["W"] if kind == "relu" else None
        entry = {"m": m}
        for causal in (False, True):
            ws = favor.Workspace(B, H, n, d, m, causal=causal, phi=kind)
            out = torch.empty((B, H, n, d), dtype=torch.float32, device=dev)

            def call(i):
                t = sets[i % len(sets)]
                favor.attention(t["q"], t["k"], t["v"], W, causal=causal, out=out, workspace=ws, phi=kind)

            for i in range(3):
                call(i)
            torch.cuda.synchronize()
            _lib.check(_lib.favor_profile_enable())
            for i in range(steps):
                call(i)
            torch.cuda.synchronize()
            prof = _lib.favor_profile_collect()
            kernels = {k: round(t / c * 1e3, 2) for k, (c, t) in prof.items()}
            us = sum(kernels.values())
            call_bytes = 10.0 * B * H * n * d + (2.0 * H * m * d if kind == "relu" else 0.0)
            dom = max(kernels, key=kernels.get)
            entry["causal" if causal else "noncausal"] = {
                "kernel_us": round(us, 2),
                "tokens_per_s": round(B * n / (us * 1e-6), 1),
                "hbm_frac": round(call_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "bytes_per_call": call_bytes,
                "dominant": dom,
                "kernels_us": kernels,
            }
            assert bool(torch.isfinite(out).all()), f"{kind} attention produced non-finite outputs"
        if cpu_budget_s > 0:
            import oracle  # cpu_baseline leg only
            x = {k: sets[0][k][0, 0].float().cpu().numpy() for k in ("q", "k", "v")}
            Wh = sets[0]["W"][0].float().cpu().numpy() if kind == "relu" else None
            slices, t0 = 0, time.perf_counter()
            while True:
                oracle.attention(x["q"], x["k"], x["v"], Wh, kind=kind)
                oracle.attention_causal(x["q"], x["k"], x["v"], Wh, kind=kind)
                slices += 1
                if time.perf_counter() - t0 >= cpu_budget_s:
                    break
            wall = time.perf_counter() - t0
            entry["cpu_baseline"] = {
                "value": round(slices * n / H / wall, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                "sample": f"{slices} whole (b,h) slice(s) of n={n} through the fp64 oracle's non-causal and "
                          f"causal {kind} attention in {wall:.1f} s, one process"}
        res[kind] = entry
    return res


# ---------------------------------------------------- random feature draws
def bench_draw(favor, _lib, torch, cfg, steps: int, cpu_budget_s: float) -> dict:
    """W [H, m, d] drawn on the device (a per-call or per-step redraw), timed
    with HIP events around each launch; the oracle's draw of the same W beside."""
    H, m, d = cfg.H, cfg.m, cfg.d
    W = torch.empty((H, m, d), dtype=torch.bfloat16, device="cuda")
    for i in range(3):
        favor.draw_features(1, i, H, m, d, out=W)
    torch.cuda.synchronize()
    _lib.check(_lib.favor_profile_enable())
    for i in range(steps):
        favor.draw_features(1, 100 + i, H, m, d, out=W)
    torch.cuda.synchronize()
    c, t = _lib.favor_profile_collect()["k_draw_features"]
    us = t / c * 1e3
    nb = (m + d - 1) // d
    # fp64 work per block: d*d*2 normals (Philox + Box-Muller, counted as 40 flops each)
    # and modified Gram-Schmidt (2 d^3)
    flops = H * nb * (2 * d * d * 40 + 2 * d ** 3)
    out = {"workload": f"H={H} m={m} d={d}, bf16 out", "kernel_us": round(us, 2),
           "fp64_gflop": round(flops / 1e9, 4),
           "fp64_frac": round(flops / (us * 1e-6) / 1e12 / FP64_PEAK_TFLOPS, 5)}
    if cpu_budget_s > 0:
        import oracle  # cpu_baseline leg only
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.draw_features(1, n, H, m, d)
            n += 1
            if time.perf_counter() - t0 >= cpu_budget_s:
                break
        wall = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(wall / n * 1e6, 1), "unit": "us per draw", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} draws of W [{H},{m},{d}] by the fp64 oracle in {wall:.1f} s"}
    return out


# ------------------------------------------------------------- backward pass
def bench_backward(favor, _lib, torch, cfg, sets, dev, steps: int, cpu_budget_s: float, causal: bool) -> dict:
    """dq, dk, dv for the workload's call (non-causal or causal): per-kernel
    HIP-event means over `steps` backward calls (the forward output computed
    once, outside), tokens/s and HBM fraction; the oracle's gradients on sampled
    rows beside."""
    B, H, n, d, m = cfg.B, cfg.H, cfg.n, cfg.d, cfg.m
    t = sets[0]
    y = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=causal)
    dy = torch.randn((B, H, n, d), generator=torch.Generator(device="cpu").manual_seed(5)).to(dev)
    nb = _lib.favor_backward_workspace_bytes(B, H, n, d, m, int(causal))
    ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
    outs = tuple(torch.empty((B, H, n, d), dtype=torch.float32, device=dev) for _ in range(3))
    for _ in range(3):
        favor.attention_backward(t["q"], t["k"], t["v"], t["W"], y, dy, causal=causal, out=outs, workspace=ws)
    torch.cuda.synchronize()
    _lib.check(_lib.favor_profile_enable())
    for _ in range(steps):
        favor.attention_backward(t["q"], t["k"], t["v"], t["W"], y, dy, causal=causal, out=outs, workspace=ws)
    torch.cuda.synchronize()
    prof = _lib.favor_profile_collect()
    kernels = {k: round(tt / c * 1e3, 2) for k, (c, tt) in prof.items()}   # mean per launch
    us = sum(tt for _, tt in prof.values()) * 1e3 / steps                    # all launches of one call
    # algorithmic bytes: q, k, v (bf16), y and dy (fp32) read once, dq, dk, dv (fp32) written once
    call_bytes = 3 * 2.0 * B * H * n * d + 2 * 4.0 * B * H * n * d + 3 * 4.0 * B * H * n * d + 2.0 * H * m * d
    assert all(bool(torch.isfinite(o).all()) for o in outs), "non-finite gradients"
    kind = "causal" if causal else "non-causal"
    # the call's dominant kernel against the HBM roof (algorithmic bytes per launch)
    dom = max(kernels, key=kernels.get)
    dbytes = kernel_bytes(dom, B, H, n, d, m)
    droof = None
    if dbytes > 0:
        ach = dbytes / (kernels[dom] * 1e-6) / 1e9
        droof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(ach / HBM_PEAK_GBS, 4), "bytes_per_launch": dbytes}
    out = {"workload": f"{kind} backward B={B} H={H} n={n} d={d} m={m}", "kernel_us": round(us, 2),
           "tokens_per_s": round(B * n / (us * 1e-6), 1), "bytes_per_call": call_bytes,
           "hbm_frac": round(call_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "kernels_us": kernels,
           "roofline": droof}
    if cpu_budget_s > 0:
        import numpy as np
        import oracle  # cpu_baseline leg only
        x = {k: t[k][0, 0].float().cpu().numpy() for k in ("q", "k", "v")}
        Wh = t["W"][0].float().cpu().numpy()
        g = dy[0, 0].cpu().numpy()
        # the causal form builds every prefix state once per call: hand it more rows per call
        per = 64 if causal else 4
        rows, t0, r0 = 0, time.perf_counter(), 0
        while True:
            sel = (r0 + np.arange(per) * max(1, n // per)) % n
            oracle.attention_backward_rows(x["q"], x["k"], x["v"], Wh, g, sel, sel, causal=causal)
            rows += per
            r0 += 1
            if time.perf_counter() - t0 >= cpu_budget_s:
                break
        wall = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(rows / H / wall, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"dq, dk, dv of {rows} rows of one (b,h) slice of n={n} through the "
                                         f"fp64 oracle's sampled-row {kind} backward in {wall:.1f} s, one process"}
    return out


# ----------------------------------------------------------- other workloads
BUDGETS_US = {"C3": 70.0, "C4": 104.9, "C5": 209.8}   # 60% of the HBM roof per call


def bench_workload(favor, torch, fi, name: str, causal: bool, dev, calls: int, sets: int = 2) -> dict:
    """One attention call per step on another workload (its own inputs, rotated
    sets, workspace pre-allocated): per-call HIP-event times on the launch
    stream (median / p10 / p90), tokens/s and HBM fraction against its budget."""
    cfg = fi.config(name)
    B, H, n, d, m = cfg.B, cfg.H, cfg.n, cfg.d, cfg.m
    xs = []
    for si in range(sets):
        x = fi.make_inputs(cfg, set_index=si)
        xs.append({k: torch.from_numpy(v).to(device=dev, dtype=torch.bfloat16) for k, v in x.items()})
        del x
    ws = favor.Workspace(B, H, n, d, m, causal=causal)
    outs = [torch.empty((B, H, n, d), dtype=torch.float32, device=dev) for _ in range(sets)]

    def call(i):
        t = xs[i % sets]
        favor.attention(t["q"], t["k"], t["v"], t["W"], causal=causal, out=outs[i % sets], workspace=ws)

    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for i in range(calls):
        ev[i][0].record()
        call(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    assert all(bool(torch.isfinite(o).all()) for o in outs), f"{name} produced non-finite outputs"
    dd = dist(us)
    call_bytes = 10.0 * B * H * n * d + 2.0 * H * m * d
    med = dd["median_us"]
    return {
        "workload": f"{name}: FAVOR+ {'causal (chunk 64)' if causal else 'non-causal'} B={B} H={H} n={n} d={d} "
                    f"m={m}" + (" (low-rank Q/K vision stand-in)" if cfg.qk == "lowrank" else ""),
        "per_call": dd,
        "tokens_per_s": round(B * n / (med * 1e-6), 1),
        "bytes_per_call": call_bytes,
        "hbm_frac": round(call_bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "budget_us": BUDGETS_US.get(name),
    }


# ------------------------------------------------------------------- main
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=3, help="independent input sets rotated between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--noncausal-only", action="store_true", help="time only the non-causal call")
    ap.add_argument("--no-decode", action="store_true", help="skip the streaming-decode measurement")
    ap.add_argument("--no-phi", action="store_true", help="skip the ReLU / elu+1 feature-map measurement")
    ap.add_argument("--no-draw", action="store_true", help="skip the on-device feature draw measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--no-workloads", action="store_true", help="skip the C4 causal and C5 vision legs")
    ap.add_argument("--no-probes", action="store_true", help="skip the instruction-rate probes")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="before timing, run a plain elementwise copy (negation) of MB MiB fp32 three "
                         "times; its HBM counters calibrate the per-kernel traffic figures")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard over (b, h) or over the sequence)", file=sys.stderr)
        return 2

    import numpy as np  # noqa: F401
    import torch

    import favor_inputs as fi
    import kernelized_linear_attention_favor_amd as favor
    from kernelized_linear_attention_favor_amd import _lib

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    cfg = fi.config("C3")
    B, H, n, d, m = cfg.B, cfg.H, cfg.n, cfg.d, cfg.m
    print(f"[bench] generating {args.sets} input sets B={B} H={H} n={n} d={d} m={m}", file=sys.stderr, flush=True)
    sets = []
    host0 = None
    for si in range(args.sets):
        x = fi.make_inputs(cfg, set_index=si)
        if si == 0:
            host0 = x
        sets.append({k: torch.from_numpy(v).to(device=dev, dtype=torch.bfloat16) for k, v in x.items()})
        if si:
            del x
    W = sets[0]["W"]
    outs_nc = [torch.empty((B, H, n, d), dtype=torch.float32, device=dev) for _ in sets]
    outs_c = [torch.empty((B, H, n, d), dtype=torch.float32, device=dev) for _ in sets]
    ws_nc = favor.Workspace(B, H, n, d, m, causal=False)
    causal_ok = not args.noncausal_only
    ws_c = None
    if causal_ok:
        try:
            ws_c = favor.Workspace(B, H, n, d, m, causal=True)
            t = sets[0]
            favor.attention(t["q"], t["k"], t["v"], W, causal=True, out=outs_c[0], workspace=ws_c)
            torch.cuda.synchronize()
        except favor.FavorError as e:
            print(f"[bench] causal path unavailable: {e}", file=sys.stderr)
            causal_ok = False

    if args.copy_probe > 0:
        nel = args.copy_probe * (1 << 20) // 4
        src = torch.randn(nel, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: {4 * nel} bytes read and {4 * nel} bytes written per launch",
              file=sys.stderr, flush=True)
        del src, dst

    def call_nc(i):
        t = sets[i % len(sets)]
        favor.attention(t["q"], t["k"], t["v"], W, causal=False, out=outs_nc[i % len(sets)], workspace=ws_nc)

    def call_c(i):
        t = sets[i % len(sets)]
        favor.attention(t["q"], t["k"], t["v"], W, causal=True, out=outs_c[i % len(sets)], workspace=ws_c)

    def step(i):
        call_nc(i)
        if causal_ok:
            call_c(i)

    # warmup (no instrumentation)
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps back to back, events only at its two ends (on the
    # stream every kernel is launched on: torch's current stream)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # per-kernel breakdown (every launch bracketed by events; outside the timed region)
    _lib.check(_lib.favor_profile_enable())
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    bprof = _lib.favor_profile_collect()
    dname = max(bprof.items(), key=lambda kv: kv[1][1])[0]

    # the dominant kernel alone bracketed (its launch stream), for the roofline
    _lib.check(_lib.favor_profile_enable_only(dname))
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dcount, dtotal = _lib.favor_profile_collect()[dname]
    avg_ms = dtotal / dcount

    # per-call distributions (events between calls only)
    calls = {"noncausal": [], "causal": []}
    for i in range(args.steps):
        for g, fn in (("noncausal", call_nc), ("causal", call_c)):
            if g == "causal" and not causal_ok:
                continue
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(i)
            b.record()
            calls[g].append((a, b))
    torch.cuda.synchronize()
    call_dist = {g: dist([a.elapsed_time(b) * 1e3 for a, b in ev]) for g, ev in calls.items() if ev}
    print(f"[bench] {ms:.4f} ms/step; {dname} {avg_ms * 1e3:.1f}us (alone bracketed); calls: "
          + json.dumps(call_dist) + "; kernels: "
          + ", ".join(f"{k} {c}x {t / c * 1e3:.1f}us" for k, (c, t) in bprof.items()),
          file=sys.stderr, flush=True)

    # the self-allocating entries: no workspace argument, so each call allocates,
    # clears and frees its scratch stream-ordered (timed the same way, for comparison)
    def step_alloc(i):
        t = sets[i % len(sets)]
        favor.attention(t["q"], t["k"], t["v"], W, causal=False, out=outs_nc[i % len(sets)])
        if causal_ok:
            favor.attention(t["q"], t["k"], t["v"], W, causal=True, out=outs_c[i % len(sets)])

    for i in range(3):
        step_alloc(i)
    torch.cuda.synchronize()
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    a0.record()
    for i in range(args.steps):
        step_alloc(i)
    a1.record()
    torch.cuda.synchronize()
    ms_alloc = a0.elapsed_time(a1) / args.steps

    tokens = B * n
    value = tokens / (ms * 1e-3)
    dbytes = kernel_bytes(dname, B, H, n, d, m)
    achieved = dbytes / (avg_ms * 1e-3) / 1e9
    digest = source_digest()
    traffic = read_traffic(dname, digest)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": dname,
        "kernel_us": round(avg_ms * 1e3, 2),
        "bytes_per_launch": dbytes,
    }
    # whole-call view: algorithmic bytes and flops of each attention call
    call_bytes = 10.0 * B * H * n * d + 2.0 * H * m * d
    call_flops = (8.0 * n * m * d + 4.0 * n * m) * B * H
    kernels = {k: {"launches": c, "mean_us": round(t / c * 1e3, 2)} for k, (c, t) in bprof.items()}
    per_call = {}
    groups = {"noncausal": ("k_kv_state", "k_merge", "k_output"),
              "causal": ("k_causal_state", "k_causal_output", "k_causal_walk", "k_slice_combine")}
    for g, names in groups.items():
        us = sum(kernels[k]["mean_us"] for k in names if k in kernels)
        if us > 0:
            per_call[g] = {
                "kernel_us": round(us, 2),
                "tokens_per_s": round(tokens / (us * 1e-6), 1),
                "hbm_frac": round(call_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "tflops": round(call_flops / (us * 1e-6) / 1e12, 2),
                "call": call_dist.get(g),
                "budget_us": BUDGETS_US["C3"],
            }

    rates = None
    if not args.no_probes:
        print("[bench] instruction-rate probes", file=sys.stderr, flush=True)
        rates = probe_rates(torch)
        print(f"[bench] rates: {json.dumps(rates)}", file=sys.stderr, flush=True)
    valu = None
    if rates:
        # the exponential floor of each exp-forming kernel: its exps at the measured rate
        valu = {"exp2_per_s": rates["exp2_per_s"], "kernels": {}}
        for k, v in kernels.items():
            ne = exps_per_launch(k, B, H, n, m)
            if ne > 0:
                fl = ne / rates["exp2_per_s"] * 1e6
                valu["kernels"][k] = {"exps_per_launch": ne, "exp_floor_us": round(fl, 2),
                                      "frac": round(fl / v["mean_us"], 4)}

    extra = None
    if not args.no_workloads:
        extra = {}
        for name, causal in (("C4", True), ("C5", False)):
            print(f"[bench] workload {name}", file=sys.stderr, flush=True)
            extra[name] = bench_workload(favor, torch, fi, name, causal, dev, calls=args.steps)
            print(f"[bench] {name}: {json.dumps(extra[name])}", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()

    dec = None
    if not args.no_decode:
        print("[bench] streaming decode", file=sys.stderr, flush=True)
        dec = bench_decode(favor, _lib, torch, fi, cfg, sets[0], dev,
                           cpu_budget_s=0.0 if args.no_cpu_baseline else 2.0)
        print(f"[bench] decode: {json.dumps(dec)}", file=sys.stderr, flush=True)

    phi = None
    if not args.no_phi:
        print("[bench] deterministic feature maps", file=sys.stderr, flush=True)
        phi = bench_phi(favor, _lib, torch, cfg, sets, dev, steps=20,
                        cpu_budget_s=0.0 if args.no_cpu_baseline else 1.0)
        print(f"[bench] feature maps: {json.dumps(phi)}", file=sys.stderr, flush=True)

    draw = None
    if not args.no_draw:
        print("[bench] feature draw", file=sys.stderr, flush=True)
        draw = bench_draw(favor, _lib, torch, cfg, steps=20, cpu_budget_s=0.0 if args.no_cpu_baseline else 1.0)
        print(f"[bench] feature draw: {json.dumps(draw)}", file=sys.stderr, flush=True)

    bwd = bwd_c = None
    if not args.no_backward:
        print("[bench] backward pass", file=sys.stderr, flush=True)
        bwd = bench_backward(favor, _lib, torch, cfg, sets, dev, steps=10,
                             cpu_budget_s=0.0 if args.no_cpu_baseline else 2.0, causal=False)
        print(f"[bench] backward: {json.dumps(bwd)}", file=sys.stderr, flush=True)
        bwd_c = bench_backward(favor, _lib, torch, cfg, sets, dev, steps=10,
                               cpu_budget_s=0.0 if args.no_cpu_baseline else 4.0, causal=True)
        print(f"[bench] causal backward: {json.dumps(bwd_c)}", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(host0, cfg, causal_ok)

    out = {
        "metric": "FAVOR+ attention tokens/sec and % MI355X roofline (n=16k, d=64, m=256)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, Q/K scaled by d^-1/4; orthogonal random W per head)",
        "config": {
            "workload": "FAVOR+ attention B=4 H=8 n=16384 d=64 m=256, bf16 in / fp32 out; step = "
                        + ("non-causal + causal (chunk 64)" if causal_ok else "non-causal only"),
            "B": B, "H": H, "n": n, "d": d, "m": m, "chunk": 64,
            "global_batch": B, "seq_len": n, "input_sets": len(sets),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_call": per_call,
        "kernels": kernels,
        "valu": valu,
        "rates": rates,
        "workloads": extra,
        "decode": dec,
        "feature_maps": phi,
        "feature_draw": draw,
        "self_alloc": {"ms_per_step": round(ms_alloc, 5), "tokens_per_s": round(tokens / (ms_alloc * 1e-3), 1),
                       "note": "the same step through the entries without a workspace argument (scratch "
                               "allocated, cleared and freed stream-ordered in every call)"},
        "backward": bwd,
        "backward_causal": bwd_c,
        "environment": environment(torch),
        "sources": digest,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
