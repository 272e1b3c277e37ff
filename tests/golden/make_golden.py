"""Write tests/golden/favor_small_f32.json from the fp64 oracle.

Calls only oracle/ (no GPU code).  The inputs are small fixed arrays built
here from exact binary fractions, so they are representable in fp32 and bf16
alike; the stored outputs are the oracle's fp64 values.

Covers (Performer notes: FAVOR+, Kernel Attention View, Normalization;
Performer for vision: How It Works, Step 2):
  phi   = feature map of q        [B,H,n,m]
  y     = non-causal FAVOR+        [B,H,n,d]
  y_c   = causal (inclusive) FAVOR+ [B,H,n,d]

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

B, H, n, d, m = 1, 2, 12, 8, 16


def exact_grid(shape, a, b, c, den, offset):
    """Entries ((a r^2 + b j + c r j + 5 s + offset) mod den - den/2) / den for row
    r, column j and leading (batch, head) index s: exact binary fractions in fp32
    and bf16 (den a power of two), different from row to row and from head to
    head."""
    *lead, rows, cols = shape
    s = np.arange(int(np.prod(lead)) if lead else 1, dtype=np.int64)[:, None, None]
    r = np.arange(rows, dtype=np.int64)[None, :, None]
    j = np.arange(cols, dtype=np.int64)[None, None, :]
    k = (a * r * r + b * j + c * r * j + 5 * s + offset) % den
    return ((k - den // 2).astype(np.float64) / den).reshape(shape)


def main():
    q = exact_grid((B, H, n, d), 3, 7, 5, 32, 3) * 2.0
    k = exact_grid((B, H, n, d), 5, 3, 9, 32, 1) * 2.0
    v = exact_grid((B, H, n, d), 7, 5, 3, 16, 5)
    W = exact_grid((H, m, d), 1, 11, 13, 32, 7) * 2.0
    out = {
        "description": "FAVOR+ on a tiny exact-binary-fraction input; fp64 oracle outputs",
        "shape": {"B": B, "H": H, "n": n, "d": d, "m": m},
        "q": q.tolist(), "k": k.tolist(), "v": v.tolist(), "W": W.tolist(),
        "phi_q": oracle.feature_map(q, W).tolist(),
        "y": oracle.attention(q, k, v, W).tolist(),
        "y_causal": oracle.attention_causal(q, k, v, W).tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "favor_small_f32.json")
    with open(path, "w") as fh:
        json.dump(out, fh)
    print("wrote", path)


if __name__ == "__main__":
    main()
