"""Whole-output oracle references for large shapes, one (b, h) slice per task.

The fp64 oracle works on one (batch, head) slice at a time here (its memory
stays bounded), and the slices are spread over a pool of worker processes on
the host cores, so that the full causal output at the benchmark shapes (tens
of seconds per slice) is compared element by element inside a test.  The pool
is forked from the test process; the workers only run NumPy, never the GPU.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

_X = None


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass


def _one(args):
    import oracle
    b, h, causal, kind = args
    q, k, v, W = _X["q"][b, h], _X["k"][b, h], _X["v"][b, h], _X["W"]
    Wh = None if W is None else W[h]
    f = oracle.attention_causal if causal else oracle.attention
    return b, h, f(q, k, v, Wh, kind=kind)


def workers() -> int:
    """Host cores this process may use, capped at 16 (a GPU machine's CPU share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def reference(x: dict, causal: bool, kind: str = "exp", slices=None) -> np.ndarray:
    """The oracle's output for every (b, h) slice in `slices` (all by default):
    an array shaped like x["q"] (slices not asked for are left as NaN)."""
    global _X
    B, H = x["q"].shape[:2]
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    _X = {"q": x["q"], "k": x["k"], "v": x["v"], "W": x.get("W")}
    out = np.full(x["q"].shape, np.nan)
    jobs = [(b, h, causal, kind) for b, h in slices]
    nw = min(workers(), len(jobs))
    try:
        if nw <= 1:
            for j in jobs:
                b, h, r = _one(j)
                out[b, h] = r
        else:
            with mp.get_context("fork").Pool(nw, initializer=_init) as pool:
                for b, h, r in pool.imap_unordered(_one, jobs):
                    out[b, h] = r
    finally:
        _X = None
    return out


def slice_errors(y: np.ndarray, ref: np.ndarray, slices) -> dict:
    """Per-slice error max|y - ref| / max|ref| (the bf16 and fp32 metric)."""
    res = {}
    for b, h in slices:
        a = float(np.max(np.abs(y[b, h].astype(np.float64) - ref[b, h])))
        res[(b, h)] = a / float(np.max(np.abs(ref[b, h])))
    return res


def _bw_rows(args):
    import oracle
    b, h, causal, qrows, krows = args
    x = _X
    return b, h, oracle.attention_backward_rows(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["W"][h],
                                                x["dy"][b, h], qrows, krows, causal=causal)


def backward_rows(x: dict, dy: np.ndarray, causal: bool, rows: dict) -> dict:
    """The oracle's (dq, dk, dv) rows for each slice in `rows` ({(b, h): row
    indices}, used for both the query and the key rows), one slice per task."""
    global _X
    _X = {"q": x["q"], "k": x["k"], "v": x["v"], "W": x["W"], "dy": dy}
    jobs = [(b, h, causal, r, r) for (b, h), r in rows.items()]
    out = {}
    try:
        nw = min(workers(), len(jobs))
        if nw <= 1:
            for j in jobs:
                b, h, r = _bw_rows(j)
                out[(b, h)] = r
        else:
            with mp.get_context("fork").Pool(nw, initializer=_init) as pool:
                for b, h, r in pool.imap_unordered(_bw_rows, jobs):
                    out[(b, h)] = r
    finally:
        _X = None
    return out
