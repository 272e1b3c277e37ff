"""fp64 CPU oracle for FAVOR+ attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never calls it and shares no code with it.
"""
from .favor_oracle import (  # noqa: F401
    feature_map, kv_state, attention, attention_causal, decode, attention_quadratic,
    attention_quadratic_rows, softmax_attention, max_rel_err, PHI_KINDS,
    philox4x64_10, draw_normals, draw_features, attention_backward,
    attention_backward_rows,
)
