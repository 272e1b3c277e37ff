"""ctypes binding for libfavor (include/favor.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libfavor.so.  The library must have been built in-tree (see
build.py); importing this module never falls back to anything else.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# Always the library build.py writes next to this file: no other build is ever loaded.
LIB_PATH = os.path.join(_HERE, "libfavor.so")

FAVOR_OK = 0
FAVOR_ERR_INVALID_ARGUMENT = 1
FAVOR_ERR_UNSUPPORTED = 2
FAVOR_ERR_HIP = 3
FAVOR_ERR_OUT_OF_MEMORY = 4

FAVOR_PHI_EXP = 0
FAVOR_PHI_RELU = 1
FAVOR_PHI_ELU1 = 2

FAVOR_OUT_BF16 = 0
FAVOR_OUT_F32 = 1

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); the same list as include/favor.h
SIGNATURES = {
    "favor_version": (_i, []),
    "favor_status_string": (ctypes.c_char_p, [_i]),
    "favor_last_error": (ctypes.c_char_p, []),
    "favor_feature_map": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "favor_feature_map_f32": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "favor_attention": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "favor_attention_causal": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "favor_attention_f32": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "favor_attention_causal_f32": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "favor_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "favor_attention_ws": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "favor_attention_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "favor_workspace_bytes_phi": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "favor_attention_phi": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "favor_draw_features": (_i, [ctypes.c_ulonglong, ctypes.c_ulonglong, _vp, _i, _i, _i, _i, _vp]),
    "favor_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "favor_attention_backward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                      _vp, _sz, _vp]),
    "favor_state_bytes": (_sz, [_i, _i, _i, _i]),
    "favor_state_reset": (_i, [_vp, _i, _i, _i, _i, _vp]),
    "favor_state_from_keys": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "favor_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "favor_profile_enable": (_i, []),
    "favor_profile_enable_only": (_i, [ctypes.c_char_p]),
    "favor_set_handover_spin_limit": (_i, [_i]),
    "favor_profile_collect": (_i, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_i),
                                   ctypes.POINTER(ctypes.c_double), _i]),
}

_lib = None


class FavorError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_string(status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfavor.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')"
            )
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().favor_status_string(st).decode()


def last_error() -> str:
    return lib().favor_last_error().decode()


def check(st: int) -> None:
    if st != FAVOR_OK:
        raise FavorError(st, last_error())


# Raw pointer-level calls with the C names (pointers and streams as ints).
def favor_version() -> int:
    return lib().favor_version()


def favor_feature_map(x, W, phi, B, H, n, d, m, stream) -> int:
    return lib().favor_feature_map(x, W, phi, B, H, n, d, m, stream)


def favor_feature_map_f32(x, W, phi, B, H, n, d, m, stream) -> int:
    return lib().favor_feature_map_f32(x, W, phi, B, H, n, d, m, stream)


def favor_attention(q, k, v, W, out, B, H, n, d, m, causal, stream) -> int:
    return lib().favor_attention(q, k, v, W, out, B, H, n, d, m, causal, stream)


def favor_attention_causal(q, k, v, W, out, B, H, n, d, m, chunk, stream) -> int:
    return lib().favor_attention_causal(q, k, v, W, out, B, H, n, d, m, chunk, stream)


def favor_attention_f32(q, k, v, W, out, B, H, n, d, m, causal, stream) -> int:
    return lib().favor_attention_f32(q, k, v, W, out, B, H, n, d, m, causal, stream)


def favor_attention_causal_f32(q, k, v, W, out, B, H, n, d, m, chunk, stream) -> int:
    return lib().favor_attention_causal_f32(q, k, v, W, out, B, H, n, d, m, chunk, stream)


def favor_workspace_bytes(B, H, n, d, m, causal) -> int:
    return lib().favor_workspace_bytes(B, H, n, d, m, causal)


def favor_attention_ws(q, k, v, W, out, B, H, n, d, m, causal, ws, ws_bytes, stream) -> int:
    return lib().favor_attention_ws(q, k, v, W, out, B, H, n, d, m, causal, ws, ws_bytes, stream)


def favor_attention_noalloc(q, k, v, W, out, B, H, n, d, m, causal, stream) -> int:
    return lib().favor_attention_noalloc(q, k, v, W, out, B, H, n, d, m, causal, stream)


def favor_workspace_bytes_phi(B, H, n, d, m, causal, phi) -> int:
    return lib().favor_workspace_bytes_phi(B, H, n, d, m, causal, phi)


def favor_attention_phi(q, k, v, W, out, B, H, n, d, m, causal, phi, ws, ws_bytes, stream) -> int:
    return lib().favor_attention_phi(q, k, v, W, out, B, H, n, d, m, causal, phi, ws, ws_bytes, stream)


def favor_draw_features(seed, step, W, out_dtype, H, m, d, stream) -> int:
    return lib().favor_draw_features(seed, step, W, out_dtype, H, m, d, stream)


def favor_backward_workspace_bytes(B, H, n, d, m, causal) -> int:
    return lib().favor_backward_workspace_bytes(B, H, n, d, m, causal)


def favor_attention_backward(q, k, v, W, y, dy, dq, dk, dv, B, H, n, d, m, causal, ws, ws_bytes, stream) -> int:
    return lib().favor_attention_backward(q, k, v, W, y, dy, dq, dk, dv, B, H, n, d, m, causal, ws, ws_bytes,
                                          stream)


def favor_state_bytes(B, H, d, m) -> int:
    return lib().favor_state_bytes(B, H, d, m)


def favor_state_reset(state, B, H, d, m, stream) -> int:
    return lib().favor_state_reset(state, B, H, d, m, stream)


def favor_state_from_keys(k, v, W, state, B, H, n, d, m, stream) -> int:
    return lib().favor_state_from_keys(k, v, W, state, B, H, n, d, m, stream)


def favor_decode(q, k, v, W, state, out, B, H, T, d, m, stream) -> int:
    return lib().favor_decode(q, k, v, W, state, out, B, H, T, d, m, stream)


def favor_profile_enable() -> int:
    return lib().favor_profile_enable()


def favor_profile_enable_only(name) -> int:
    return lib().favor_profile_enable_only(None if name is None else name.encode())


def favor_set_handover_spin_limit(limit) -> int:
    return lib().favor_set_handover_spin_limit(limit)


def favor_profile_collect(capacity: int = 32) -> dict:
    """{kernel name: (launch count, total ms)} for launches since favor_profile_enable()."""
    names = (ctypes.c_char_p * capacity)()
    counts = (_i * capacity)()
    tot = (ctypes.c_double * capacity)()
    k = lib().favor_profile_collect(names, counts, tot, capacity)
    if k < 0:
        raise FavorError(FAVOR_ERR_HIP, "HIP event failure while collecting kernel timings")
    return {names[i].decode(): (counts[i], tot[i]) for i in range(min(k, capacity))}
