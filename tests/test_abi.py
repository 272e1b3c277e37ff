"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "favor.h")


def _lib():
    from kernelized_linear_attention_favor_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libfavor.so not built")
    return _lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(favor_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("favor_feature_map", "favor_attention", "favor_attention_causal",
              "favor_attention_ws", "favor_workspace_bytes", "favor_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    raw = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(declared_functions()) == set(L.SIGNATURES)


UBENCH_HEADER = os.path.join(ROOT, "include", "favor_ubench.h")
UBENCH_LIB = os.path.join(ROOT, "kernelized_linear_attention_favor_amd", "libfavor_ubench.so")


def test_probe_library_exports_its_header():
    """The instruction-rate probes (bench.py's measurements) are a library of
    their own; it exports what its header declares and rejects bad launches."""
    if not os.path.exists(UBENCH_LIB):
        pytest.skip("libfavor_ubench.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(UBENCH_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(favor_ubench_[a-z0-9_]+)\s*\(", text)))
    assert names == ["favor_ubench_exp2", "favor_ubench_fma", "favor_ubench_mix"]
    raw = ctypes.CDLL(UBENCH_LIB)
    for name in names:
        fn = getattr(raw, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        assert fn(None, 1, 64, 1, None) == 1          # null out
        assert fn(0x100000, 1, 96, 1, None) == 1      # threads not a multiple of 64
        assert fn(0x100000, 1, 64, 0, None) == 1      # no iterations


def test_version_and_status_strings():
    L = _lib()
    assert L.favor_version() == 10000
    assert L.status_string(0) == "FAVOR_OK"
    assert L.status_string(2) == "FAVOR_ERR_UNSUPPORTED"
    assert L.status_string(99) == "FAVOR_ERR_UNKNOWN"


def test_workspace_bytes_host_only():
    L = _lib()
    assert L.favor_workspace_bytes(4, 8, 16384, 64, 256, 0) > 0
    assert L.favor_workspace_bytes(4, 8, 16384, 64, 256, 1) > 0
    # the bf16 path: d in {32, 64}, every m in 16Z from 16 to 512
    for d in (32, 64):
        for m in range(16, 513, 16):
            for causal in (0, 1):
                assert L.favor_workspace_bytes(2, 3, 1000, d, m, causal) > 0, (d, m, causal)
    assert L.favor_workspace_bytes(4, 8, 16384, 48, 256, 0) == 0   # d unsupported
    assert L.favor_workspace_bytes(4, 8, 16384, 128, 256, 0) == 0  # d unsupported
    assert L.favor_workspace_bytes(4, 8, 16384, 64, 100, 0) == 0   # m not a multiple of 16
    assert L.favor_workspace_bytes(4, 8, 16384, 64, 8, 0) == 0     # m below 16
    assert L.favor_workspace_bytes(4, 8, 16384, 64, 528, 0) == 0   # m above 512
    assert L.favor_workspace_bytes(0, 8, 16384, 64, 256, 0) == 0
    assert L.favor_workspace_bytes(1, 1, 16, 64, 64, 2) == 0


FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails validation


@pytest.mark.parametrize("args,status", [
    ((0, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 64, 0), 1),        # null q
    ((FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 16, 64, 64, 0), 1),        # null out
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 16, 64, 64, 0), 1),     # B = 0
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, -3, 64, 64, 0), 1),     # n < 0
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 64, 2), 1),     # causal flag
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 48, 64, 0), 2),     # d unsupported
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 16, 64, 0), 2),     # d unsupported
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 100, 0), 2),    # m not a multiple of 16
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 528, 0), 2),    # m above 512
    ((FAKE + 2, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 64, 0), 2),  # misaligned
])
def test_attention_rejects_bad_arguments(args, status):
    L = _lib()
    st = L.favor_attention(*args, None)
    assert st == status
    assert L.last_error() != ""


def test_causal_chunk_and_f32_limits():
    L = _lib()
    base = (FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 64)
    for bad in (8, 24, 48, 96, 256):
        assert L.favor_attention_causal(*base, bad, None) == 2, bad   # chunk not in {16, 32, 64, 128}
    assert L.favor_attention_causal(*base, -1, None) == 1
    assert L.favor_attention_causal(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 100, 32, None) == 2
    assert L.favor_attention_f32(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 256, 64, 0, None) == 2
    assert L.favor_attention_f32(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 1024, 0, None) == 2
    assert L.favor_feature_map(0, FAKE, FAKE, 1, 1, 16, 64, 64, None) == 1
    assert L.favor_feature_map(FAKE, FAKE, FAKE, 1, 1, 16, 512, 64, None) == 2
    assert L.favor_attention_ws(*base, 0, 0, 0, None) == 1
    assert L.favor_attention_ws(*base, 0, FAKE, 16, None) == 4   # workspace too small


def test_no_cpu_path():
    import torch
    import kernelized_linear_attention_favor_amd as favor
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    W = torch.zeros(1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        favor.attention(q, q, q, W)


def test_profile_filter_host_only():
    # no kernel is launched: the hooks record nothing and collect reports 0 kernels
    L = _lib()
    assert L.favor_profile_enable_only("k" * 80) == 1   # name too long
    assert L.favor_profile_enable_only("k_output") == 0
    assert L.favor_profile_collect() == {}
    assert L.favor_profile_enable_only(None) == 0
    assert L.favor_profile_collect() == {}


def test_handover_spin_limit_host_only():
    # the causal kernel's hand-over wait limit: a setting only, no launch
    L = _lib()
    assert L.favor_set_handover_spin_limit(-1) == 1   # invalid argument
    assert L.favor_set_handover_spin_limit(0) == 0
    assert L.favor_set_handover_spin_limit(4096) == 0


def test_decode_entries_host_only():
    L = _lib()
    assert L.favor_state_bytes(2, 3, 64, 256) == 4 * 2 * 3 * (256 * (64 + 2) + 1)
    assert L.favor_state_bytes(1, 1, 32, 256) == 0      # d != 64
    assert L.favor_state_bytes(1, 1, 64, 100) == 0      # m not in {64,128,256}
    assert L.favor_state_reset(None, 1, 1, 64, 64, None) == 1
    assert L.favor_state_reset(FAKE, 1, 1, 64, 96, None) == 2
    assert L.favor_state_reset(FAKE, 0, 1, 64, 64, None) == 1
    base = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.favor_decode(*base, 1, 1, 0, 64, 64, None) == 1          # T = 0
    assert L.favor_decode(*base, 1, 1, 4, 48, 64, None) == 2          # d unsupported
    assert L.favor_decode(None, *base[1:], 1, 1, 4, 64, 64, None) == 1
    assert L.favor_state_from_keys(FAKE, FAKE, FAKE, None, 1, 1, 8, 64, 64, None) == 1
    assert L.favor_state_from_keys(FAKE, FAKE, FAKE, FAKE, 1, 1, 0, 64, 64, None) == 1


def test_feature_map_kinds_host_only():
    L = _lib()
    # scratch sizes: the exp map forwards to the FAVOR+ path; ReLU and elu+1 have their own plan
    assert L.favor_workspace_bytes_phi(4, 8, 16384, 64, 256, 0, 0) == L.favor_workspace_bytes(4, 8, 16384, 64, 256, 0)
    for causal in (0, 1):
        assert L.favor_workspace_bytes_phi(4, 8, 16384, 64, 256, causal, 1) > 0
        assert L.favor_workspace_bytes_phi(4, 8, 16384, 64, 64, causal, 2) > 0
    assert L.favor_workspace_bytes_phi(1, 1, 64, 64, 128, 0, 2) == 0     # elu+1 needs m = d
    assert L.favor_workspace_bytes_phi(1, 1, 64, 32, 32, 0, 2) == 0      # d must be 64
    assert L.favor_workspace_bytes_phi(1, 1, 64, 64, 100, 0, 1) == 0     # m unsupported
    assert L.favor_workspace_bytes_phi(1, 1, 64, 64, 64, 0, 3) == 0      # unknown map
    assert L.favor_workspace_bytes_phi(1, 1, 64, 64, 64, 2, 1) == 0      # causal not 0/1
    F = FAKE
    args = lambda W, m, causal, phi: (F, F, F, W, F, 1, 2, 64, 64, m, causal, phi, None, 0, None)
    assert L.favor_attention_phi(*args(F, 64, 0, 3)) == L.FAVOR_ERR_INVALID_ARGUMENT
    assert L.favor_attention_phi(*args(F, 64, 0, -1)) == L.FAVOR_ERR_INVALID_ARGUMENT
    assert L.favor_attention_phi(*args(F, 64, 2, 1)) == L.FAVOR_ERR_INVALID_ARGUMENT
    assert L.favor_attention_phi(*args(None, 64, 0, 1)) == L.FAVOR_ERR_INVALID_ARGUMENT   # ReLU needs W
    assert L.favor_attention_phi(*args(F, 128, 0, 2)) == L.FAVOR_ERR_UNSUPPORTED          # elu+1: m = d
    assert L.favor_attention_phi(*args(F, 96, 0, 1)) == L.FAVOR_ERR_UNSUPPORTED
    assert L.favor_attention_phi(F + 8, F, F, F, F, 1, 2, 64, 64, 64, 0, 1, None, 0, None) == L.FAVOR_ERR_UNSUPPORTED
    assert "feature map" in L.last_error() or "aligned" in L.last_error()
    # an undersized workspace is refused before any launch
    assert L.favor_attention_phi(F, F, F, F, F, 1, 2, 64, 64, 64, 0, 1, F, 16, None) == L.FAVOR_ERR_OUT_OF_MEMORY


def test_draw_features_host_only():
    L = _lib()
    F = FAKE
    assert L.favor_draw_features(1, 0, None, 0, 8, 256, 64, None) == L.FAVOR_ERR_INVALID_ARGUMENT
    assert L.favor_draw_features(1, 0, F, 2, 8, 256, 64, None) == L.FAVOR_ERR_INVALID_ARGUMENT
    assert L.favor_draw_features(1, 0, F, 0, 0, 256, 64, None) == L.FAVOR_ERR_INVALID_ARGUMENT
    assert L.favor_draw_features(1, 0, F, 0, 8, 0, 64, None) == L.FAVOR_ERR_INVALID_ARGUMENT
    assert L.favor_draw_features(1, 0, F, 1, 8, 256, 48, None) == L.FAVOR_ERR_UNSUPPORTED
    assert L.favor_draw_features(1, 0, F + 2, 0, 8, 256, 64, None) == L.FAVOR_ERR_UNSUPPORTED
    assert "aligned" in L.last_error()


def test_backward_host_only():
    L = _lib()
    assert L.favor_backward_workspace_bytes(4, 8, 16384, 64, 256, 0) > 0
    assert L.favor_backward_workspace_bytes(4, 8, 16384, 64, 100, 0) == 0
    assert L.favor_backward_workspace_bytes(4, 8, 16384, 32, 64, 0) == 0
    assert L.favor_backward_workspace_bytes(4, 8, 16384, 64, 96, 0) == 0   # its own fixed shape set
    # the causal pass keeps both partial states (no merged tiles)
    assert L.favor_backward_workspace_bytes(4, 8, 16384, 64, 256, 1) > 0
    assert L.favor_backward_workspace_bytes(4, 8, 16384, 64, 256, 2) == 0
    F = FAKE
    ok = [F] * 9 + [1, 2, 64, 64, 64]
    assert L.favor_attention_backward(*ok, 2, None, 0, None) == L.FAVOR_ERR_INVALID_ARGUMENT
    bad_y = [F] * 4 + [None] + [F] * 4 + [1, 2, 64, 64, 64]
    assert L.favor_attention_backward(*bad_y, 0, None, 0, None) == L.FAVOR_ERR_INVALID_ARGUMENT
    odd = [F] * 5 + [F + 4] + [F] * 3 + [1, 2, 64, 64, 64]
    assert L.favor_attention_backward(*odd, 0, None, 0, None) == L.FAVOR_ERR_UNSUPPORTED
    assert L.favor_attention_backward(*([F] * 9 + [1, 2, 64, 64, 96]), 0, None, 0, None) == L.FAVOR_ERR_UNSUPPORTED
    assert L.favor_attention_backward(*([F] * 9 + [1, 2, 64, 64, 64]), 0, F, 16, None) == L.FAVOR_ERR_OUT_OF_MEMORY
    assert L.favor_attention_backward(*([F] * 9 + [1, 2, 64, 64, 64]), 1, F, 16, None) == L.FAVOR_ERR_OUT_OF_MEMORY
