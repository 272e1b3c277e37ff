"""favor_attention_noalloc (the entry for callers that cannot allocate) against
favor_attention on the same inputs: the same kernels over a fixed scratch array
instead of stream-ordered scratch, so the outputs must be bitwise equal.  Two
calls in a row, the second on a smaller input (the array keeps the first call's
contents), non-causal and causal, through the C ABI."""
import numpy as np
import pytest

import favor_inputs as fi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import kernelized_linear_attention_favor_amd as favor  # noqa: E402
from kernelized_linear_attention_favor_amd import _lib  # noqa: E402

DEV = torch.device("cuda:0")


def _inputs(B, H, n, m, seed):
    x = fi.make_inputs(fi.Config("na", B, H, n, 64, m, "bf16", False, 64, "iid", seed))
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(device=DEV, dtype=torch.bfloat16) for k, v in x.items()}


def _noalloc(t, causal):
    B, H, n, d = t["q"].shape
    m = t["W"].shape[1]
    out = torch.full((B, H, n, d), float("nan"), dtype=torch.float32, device=DEV)
    st = _lib.favor_attention_noalloc(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["W"].data_ptr(),
                                      out.data_ptr(), B, H, n, d, m, int(causal),
                                      torch.cuda.current_stream().cuda_stream)
    _lib.check(st)
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_favor_attention_twice(causal):
    big = _inputs(4, 8, 16384, 256, 71)       # the benchmark shape
    small = _inputs(1, 3, 1000, 128, 72)      # smaller: fewer ranges, other m
    for t in (big, small):
        want = favor.attention(t["q"], t["k"], t["v"], t["W"], causal=causal)
        got = _noalloc(t, causal)
        torch.cuda.synchronize()
        assert torch.equal(got, want), float((got - want).abs().max())


def test_noalloc_rejects_shape_over_its_array():
    # B*H*n large enough that the scratch needs more than the fixed 64 MiB: refused
    # before anything is launched (nothing is allocated either)
    B, H, n = 64, 64, 4096
    assert _lib.favor_workspace_bytes(B, H, n, 64, 256, 0) > (64 << 20)
    fake = 0x100000
    st = _lib.favor_attention_noalloc(fake, fake, fake, fake, fake, B, H, n, 64, 256, 0, None)
    assert st == _lib.FAVOR_ERR_UNSUPPORTED
    assert "64" in _lib.last_error() or "scratch" in _lib.last_error()
