"""FAVOR+ (Performer) linear attention for AMD MI355X, on libfavor's HIP kernels.

PyTorch supplies device memory and the current stream; every step of the
computation runs in libfavor.so.  Tensors must live on a ROCm GPU: there is no
CPU path, and calls on CPU tensors raise.

    y = attention(q, k, v, W)                  # non-causal, bf16 or fp32 inputs
    y = attention(q, k, v, W, causal=True)     # causal (prefix-sum form)
    phi = feature_map(x, W)                    # exp(W x - |x|^2/2) / sqrt(m)
    st = State(B, H, d, m); st.from_keys(k, v, W)   # streaming decode: state of a prompt,
    y = decode(q1, k1, v1, W, st)              # then T new tokens at a time (bf16)

Layouts: q, k, v, x [B, H, n, d]; W [H, m, d]; outputs float32.  The bf16
attention takes d in {32, 64} and m any multiple of 16 from 16 to 512.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import FavorError, check  # noqa: F401

__all__ = ["feature_map", "attention", "attention_causal", "Workspace", "FavorError",
           "workspace_bytes", "version", "State", "decode", "draw_features", "PHI", "attention_backward"]


def version() -> int:
    return _lib.favor_version()


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libfavor has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shapes(q: torch.Tensor, W: torch.Tensor):
    if q.dim() != 4 or W.dim() != 3:
        raise ValueError("expected q/k/v of shape [B, H, n, d] and W of shape [H, m, d]")
    B, H, n, d = q.shape
    H2, m, d2 = W.shape
    if H2 != H or d2 != d:
        raise ValueError(f"W shape {tuple(W.shape)} does not match q shape {tuple(q.shape)}")
    return B, H, n, d, m


def feature_map(x: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """phi = exp(W x - |x|^2/2)/sqrt(m) as float32 [B, H, n, m] (no stabilising shift)."""
    B, H, n, d, m = _shapes(x, W)
    dt = x.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be bfloat16 or float32")
    _need(x, "x", dt, (B, H, n, d))
    _need(W, "W", dt, (H, m, d))
    if out is None:
        out = torch.empty((B, H, n, m), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (B, H, n, m))
    fn = _lib.favor_feature_map if dt == torch.bfloat16 else _lib.favor_feature_map_f32
    check(fn(x.data_ptr(), W.data_ptr(), out.data_ptr(), B, H, n, d, m, _stream_handle(stream)))
    return out


def workspace_bytes(B: int, H: int, n: int, d: int, m: int, causal: bool = False) -> int:
    return _lib.favor_workspace_bytes(B, H, n, d, m, int(bool(causal)))


PHI = {"exp": _lib.FAVOR_PHI_EXP, "relu": _lib.FAVOR_PHI_RELU, "elu1": _lib.FAVOR_PHI_ELU1}


def _phi_code(phi: str) -> int:
    if phi not in PHI:
        raise ValueError(f"phi must be one of {sorted(PHI)} (got {phi!r})")
    return PHI[phi]


class Workspace:
    """Caller-owned scratch for the bf16 attention path (zero-filled once), for
    one feature map phi ("exp" FAVOR+, "relu", "elu1")."""

    def __init__(self, B: int, H: int, n: int, d: int, m: int, causal: bool = False,
                 device="cuda", phi: str = "exp"):
        nbytes = _lib.favor_workspace_bytes_phi(B, H, n, d, m, int(bool(causal)), _phi_code(phi))
        if nbytes == 0:
            raise FavorError(_lib.FAVOR_ERR_UNSUPPORTED, "shape not supported by the bf16 path")
        self.nbytes = nbytes
        self.phi = phi
        self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, W: torch.Tensor | None,
              causal: bool = False, out: torch.Tensor | None = None,
              workspace: Workspace | None = None, stream=None, phi: str = "exp") -> torch.Tensor:
    """Linear attention y = phi(Q) S / (phi(Q) z), float32 [B, H, n, d].

    phi "exp" is FAVOR+ (bf16 or float32 inputs); "relu" (ReLU features of W)
    and "elu1" (elu(x) + 1, m = d, W unused and may be None) take bf16 inputs."""
    if phi != "exp":
        return _attention_phi(q, k, v, W, causal, out, workspace, stream, _phi_code(phi))
    B, H, n, d, m = _shapes(q, W)
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, dt, (B, H, n, d))
    _need(W, "W", dt, (H, m, d))
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, n, d))
    s = _stream_handle(stream)
    c = int(bool(causal))
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), out.data_ptr())
    if dt == torch.float32:
        check(_lib.favor_attention_f32(*ptrs, B, H, n, d, m, c, s))
    elif workspace is not None:
        check(_lib.favor_attention_ws(*ptrs, B, H, n, d, m, c, workspace.buf.data_ptr(),
                                      workspace.nbytes, s))
    else:
        check(_lib.favor_attention(*ptrs, B, H, n, d, m, c, s))
    return out


def _attention_phi(q, k, v, W, causal, out, workspace, stream, code):
    if q.dim() != 4:
        raise ValueError("expected q/k/v of shape [B, H, n, d]")
    B, H, n, d = q.shape
    if code == _lib.FAVOR_PHI_ELU1 and W is None:
        m, wp = d, 0
    elif W is None:
        raise ValueError("this feature map needs W [H, m, d]")
    else:
        B, H, n, d, m = _shapes(q, W)
        _need(W, "W", torch.bfloat16, (H, m, d))
        wp = W.data_ptr()
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, (B, H, n, d))
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, n, d))
    ws, wsb = (workspace.buf.data_ptr(), workspace.nbytes) if workspace is not None else (None, 0)
    check(_lib.favor_attention_phi(q.data_ptr(), k.data_ptr(), v.data_ptr(), wp, out.data_ptr(), B, H, n, d, m,
                                   int(bool(causal)), code, ws, wsb, _stream_handle(stream)))
    return out


def attention_causal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, W: torch.Tensor,
                     chunk: int = 0, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Causal FAVOR+ by chunked prefix sums: chunk in {16, 32, 64, 128}, 0 = the default (64)."""
    B, H, n, d, m = _shapes(q, W)
    dt = q.dtype
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, dt, (B, H, n, d))
    _need(W, "W", dt, (H, m, d))
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, n, d))
    s = _stream_handle(stream)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), out.data_ptr())
    if dt == torch.float32:
        check(_lib.favor_attention_causal_f32(*ptrs, B, H, n, d, m, chunk, s))
    elif dt == torch.bfloat16:
        check(_lib.favor_attention_causal(*ptrs, B, H, n, d, m, chunk, s))
    else:
        raise TypeError("q must be bfloat16 or float32")
    return out


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, W: torch.Tensor, y: torch.Tensor,
                       dy: torch.Tensor, causal: bool = False, out=None, workspace: torch.Tensor | None = None,
                       stream=None):
    """Gradients (dq, dk, dv), float32 [B, H, n, d], of FAVOR+ attention for the
    upstream gradient dy, given the forward output y (bf16 q, k, v, W)."""
    B, H, n, d, m = _shapes(q, W)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, (B, H, n, d))
    _need(W, "W", torch.bfloat16, (H, m, d))
    _need(y, "y", torch.float32, (B, H, n, d))
    _need(dy, "dy", torch.float32, (B, H, n, d))
    if out is None:
        out = tuple(torch.empty((B, H, n, d), dtype=torch.float32, device=q.device) for _ in range(3))
    for t, name in zip(out, ("dq", "dk", "dv")):
        _need(t, name, torch.float32, (B, H, n, d))
    ws, wsb = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) if workspace is not None \
        else (None, 0)
    check(_lib.favor_attention_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), y.data_ptr(),
                                        dy.data_ptr(), out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
                                        B, H, n, d, m, int(bool(causal)), ws, wsb, _stream_handle(stream)))
    return out


def draw_features(seed: int, step: int, H: int, m: int, d: int, dtype=torch.bfloat16,
                  out: torch.Tensor | None = None, device="cuda", stream=None) -> torch.Tensor:
    """Orthogonal random features W [H, m, d] drawn on the device for the key
    (seed, step) (bfloat16 or float32): a new step is an independent redraw."""
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((H, m, d), dtype=dtype, device=device)
    _need(out, "out", dtype, (H, m, d))
    code = _lib.FAVOR_OUT_F32 if dtype == torch.float32 else _lib.FAVOR_OUT_BF16
    check(_lib.favor_draw_features(int(seed) & (2**64 - 1), int(step) & (2**64 - 1), out.data_ptr(), code,
                                   H, m, d, _stream_handle(stream)))
    return out


class State:
    """Streaming-decode state (fp32): S [B,H,m,d], z [B,H,m], c [B,H,m] and one
    bookkeeping word per (b, h) in one buffer, starting empty.  The carried
    prefix sums of the causal path."""

    def __init__(self, B: int, H: int, d: int, m: int, device="cuda", stream=None):
        nbytes = _lib.favor_state_bytes(B, H, d, m)
        if nbytes == 0:
            raise FavorError(_lib.FAVOR_ERR_UNSUPPORTED, "shape not supported by the decode path")
        self.B, self.H, self.d, self.m = B, H, d, m
        self.buf = torch.empty(nbytes // 4, dtype=torch.float32, device=device)
        self.reset(stream)

    def reset(self, stream=None) -> "State":
        check(_lib.favor_state_reset(self.buf.data_ptr(), self.B, self.H, self.d, self.m,
                                     _stream_handle(stream)))
        return self

    def from_keys(self, k: torch.Tensor, v: torch.Tensor, W: torch.Tensor, stream=None) -> "State":
        """Replace the state by that of the keys k, v ([B,H,n,d], bf16)."""
        B, H, n, d, m = _shapes(k, W)
        if (B, H, d, m) != (self.B, self.H, self.d, self.m):
            raise ValueError("k/W shapes do not match the state")
        _need(k, "k", torch.bfloat16, (B, H, n, d))
        _need(v, "v", torch.bfloat16, (B, H, n, d))
        _need(W, "W", torch.bfloat16, (H, m, d))
        check(_lib.favor_state_from_keys(k.data_ptr(), v.data_ptr(), W.data_ptr(), self.buf.data_ptr(),
                                         B, H, n, d, m, _stream_handle(stream)))
        return self

    def tensors(self):
        """Views (S [B,H,m,d], z [B,H,m], c [B,H,m]) of the buffer."""
        B, H, d, m = self.B, self.H, self.d, self.m
        ns, nz = B * H * m * d, B * H * m
        return (self.buf[:ns].view(B, H, m, d), self.buf[ns:ns + nz].view(B, H, m),
                self.buf[ns + nz:ns + 2 * nz].view(B, H, m))


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, W: torch.Tensor, state: State,
           out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """T new tokens (q, k, v [B,H,T,d], bf16): each joins the state in order and
    reads it (inclusive); returns y float32 [B,H,T,d] and updates the state."""
    B, H, T, d, m = _shapes(q, W)
    if (B, H, d, m) != (state.B, state.H, state.d, state.m):
        raise ValueError("q/W shapes do not match the state")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, (B, H, T, d))
    _need(W, "W", torch.bfloat16, (H, m, d))
    if out is None:
        out = torch.empty((B, H, T, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, H, T, d))
    check(_lib.favor_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), state.buf.data_ptr(),
                            out.data_ptr(), B, H, T, d, m, _stream_handle(stream)))
    return out
