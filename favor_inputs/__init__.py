"""Seeded synthetic inputs for FAVOR+ attention.

This module is shared by the tests, the benchmark and the smoke check. It draws
random numbers and converts formats; it holds none of the attention arithmetic.
The random projection matrix W is drawn here too: the FAVOR+ estimator needs a
random W, and the library takes it as an input.

Workloads (shapes and value distributions) follow the five configurations the
library is measured on:

  C1  fp32,  B=1,  H=1,  n=256,   d=32, m=64   (non-causal)
  C2  bf16,  B=1,  H=8,  n=1024,  d=64, m=256  (non-causal; also compared with softmax)
  C3  bf16,  B=4,  H=8,  n=16384, d=64, m=256  (non-causal; the measured shape)
  C4  bf16,  B=2,  H=12, n=32768, d=64, m=256  (causal, chunk 64)
  C5  bf16,  B=32, H=12, n=4096,  d=64, m=128  (non-causal, vision-style low-rank Q/K)

Q and K entries are N(0,1) (drawn in float32) scaled by d^(-1/4) (so q.k already carries the
1/sqrt(d) softmax temperature); V entries are N(0,1). The vision workload draws
Q and K as a rank-16 product plus 0.1 N(0,1) noise before the same scaling.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Config", "CONFIGS", "config", "orthogonal_W", "iid_W", "round_bf16", "bf16_bits",
    "bits_to_f32", "make_inputs", "draw_qk", "draw_v",
]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    n: int
    d: int
    m: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    chunk: int
    qk: str             # "iid" or "lowrank"
    seed: int

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def shape(self):
        return (self.B, self.H, self.n, self.d)


CONFIGS = {
    "C1": Config("C1", 1, 1, 256, 32, 64, "f32", False, 64, "iid", 1),
    "C2": Config("C2", 1, 8, 1024, 64, 256, "bf16", False, 64, "iid", 2),
    "C3": Config("C3", 4, 8, 16384, 64, 256, "bf16", False, 64, "iid", 3),
    "C4": Config("C4", 2, 12, 32768, 64, 256, "bf16", True, 64, "iid", 4),
    "C5": Config("C5", 32, 12, 4096, 64, 128, "bf16", False, 64, "lowrank", 5),
}


def config(name: str, **overrides) -> Config:
    c = CONFIGS[name]
    return c.replace(**overrides) if overrides else c


# ---------------------------------------------------------------- bf16 format
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), returned as float32.

    Non-float32 input is first converted to float32 (round to nearest even).
    The result is exactly representable in bf16, so the same numbers can be
    handed to the device (as bits) and to a CPU checker (as floats).  NaN stays
    NaN and infinities stay infinite.
    """
    f = np.array(x, dtype=np.float32, copy=True, order="C")
    u = f.view(np.uint32)
    nan = np.isnan(f)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    del lsb
    u &= np.uint32(0xFFFF0000)
    if nan.any():
        u[nan] = np.uint32(0x7FC00000)
    return f


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of values that are already bf16-representable."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------- random draws
def orthogonal_W(rng: np.random.Generator, H: int, m: int, d: int) -> np.ndarray:
    """Orthogonal random features, one independent draw per head: [H, m, d] fp64.

    Each head stacks ceil(m/d) blocks; a block is the d orthonormal rows of the
    Q factor of a d x d standard Gaussian matrix (column signs fixed by the
    signs of R's diagonal so that the block is Haar-distributed).  The stack
    is cut to m rows and row i is rescaled to the norm of a fresh N(0, I_d)
    vector, so every row is marginally N(0, I_d) while rows in one block stay
    mutually orthogonal (Performer notes, section FAVOR+; Performer for vision,
    Kernel Choices / Orthogonal Features).
    """
    nb = -(-m // d)
    W = np.empty((H, m, d), dtype=np.float64)
    for h in range(H):
        rows = []
        for _ in range(nb):
            G = rng.standard_normal((d, d))
            Qf, R = np.linalg.qr(G)
            Qf = Qf * np.sign(np.diag(R))[None, :]
            rows.append(Qf.T)
        Bk = np.concatenate(rows, axis=0)[:m]
        s = np.linalg.norm(rng.standard_normal((m, d)), axis=1)
        W[h] = Bk * s[:, None]
    return W


def iid_W(rng: np.random.Generator, H: int, m: int, d: int) -> np.ndarray:
    """Unstructured Gaussian features (rows iid N(0, I_d)): [H, m, d] fp64."""
    return rng.standard_normal((H, m, d))


def draw_qk(rng: np.random.Generator, B: int, H: int, n: int, d: int, kind: str) -> np.ndarray:
    """Q or K as float32 [B, H, n, d], already multiplied by d^(-1/4).

    kind "iid": entries N(0, 1).  kind "lowrank": A B^T / sqrt(16) + 0.1 E with
    A [n, 16], B [d, 16], E [n, d] all N(0, 1), drawn per (b, h).
    """
    f32 = np.float32
    if kind == "iid":
        X = rng.standard_normal((B, H, n, d), dtype=f32)
    elif kind == "lowrank":
        r = 16
        A = rng.standard_normal((B, H, n, r), dtype=f32)
        Bf = rng.standard_normal((B, H, d, r), dtype=f32)
        X = np.matmul(A, np.swapaxes(Bf, -1, -2))
        X *= f32(1.0 / math.sqrt(r))
        E = rng.standard_normal((B, H, n, d), dtype=f32)
        E *= f32(0.1)
        X += E
        del E
    else:
        raise ValueError(kind)
    X *= f32(d ** -0.25)
    return X


def draw_v(rng: np.random.Generator, B: int, H: int, n: int, d: int) -> np.ndarray:
    return rng.standard_normal((B, H, n, d), dtype=np.float32)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        if x.dtype == np.float32 and x.flags.c_contiguous:
            f = x.view(np.uint32)  # round in place: x is a fresh draw owned by the caller
            nan = np.isnan(x)
            lsb = (f >> 16) & np.uint32(1)
            f += np.uint32(0x7FFF)
            f += lsb
            del lsb
            f &= np.uint32(0xFFFF0000)
            if nan.any():
                f[nan] = np.uint32(0x7FC00000)
            return x
        return round_bf16(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def make_inputs(cfg: Config, *, qk_scale: float = 1.0, w_kind: str = "orthogonal",
                set_index: int = 0) -> dict:
    """Seeded inputs for one configuration.

    Returns float32 arrays q, k, v [B,H,n,d] and W [H,m,d] whose values are
    exactly representable in cfg.dtype (bf16 values are stored widened to
    float32).  Child streams of SeedSequence(seed) feed W, Q, K and V in that
    order.  qk_scale multiplies Q and K before rounding (stress inputs).
    set_index selects an independent input set of the same shape.
    """
    ss = np.random.SeedSequence([cfg.seed, set_index])
    rw, rq, rk, rv = (np.random.default_rng(s) for s in ss.spawn(4))
    if w_kind == "orthogonal":
        W = orthogonal_W(rw, cfg.H, cfg.m, cfg.d)
    elif w_kind == "iid":
        W = iid_W(rw, cfg.H, cfg.m, cfg.d)
    else:
        raise ValueError(w_kind)
    out = {"W": _cast(W, cfg.dtype)}
    for name, r in (("q", rq), ("k", rk)):
        X = draw_qk(r, cfg.B, cfg.H, cfg.n, cfg.d, cfg.qk)
        if qk_scale != 1.0:
            X *= np.float32(qk_scale)
        out[name] = _cast(X, cfg.dtype)
        del X
    out["v"] = _cast(draw_v(rv, cfg.B, cfg.H, cfg.n, cfg.d), cfg.dtype)
    return out
