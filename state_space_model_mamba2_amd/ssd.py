"""Python face of libssd: the Mamba-2 SSD chunked scan, forward and backward.

    y, final_state, ctx = fwd(x, dt, A, B, C, D, chunk, initial_state=None,
                              dt_softplus=False, dt_bias=None)
    grads = bwd(dy, ctx, dfinal_state=None)   # dict: dx, ddt, dA, dB, dC, dD
                                              # (+ dinitial_state on request,
                                              #  + ddt_bias with dt_softplus)

Tensors are torch tensors on the GPU (torch supplies device memory and the
stream).  Every step of the computation runs in libssd's HIP kernels; this
module only checks dtypes/contiguity, allocates outputs and workspaces and
passes pointers.  It raises if libssd.so has not been built.

Layouts: x, y, dx, dy [b, L, H, P]; dt, ddt [b, L, H]; B, C, dB, dC [b, L, G, N];
A, D, dA, dD [H] float32; final_state, initial_state, dfinal_state and
dinitial_state [b, H, P, N] float32.  x, dt, B, C, dy share one dtype
(torch.bfloat16 or torch.float32).
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.SSD_F32, torch.bfloat16: _lib.SSD_BF16, torch.float8_e4m3fn: _lib.SSD_FP8}
_ALIGN = 256


def _check(code: int, what: str):
    if code != _lib.SSD_OK:
        raise RuntimeError(f"{what} failed: {_lib.status_string(code)} (status {code})")


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


@dataclasses.dataclass
class Context:
    """What the backward needs from the forward: the borrowed inputs, the
    saved workspace (per-chunk cumsums and chunk-entry states) and the C
    struct pointing at them.  Keeps every referenced tensor alive."""
    saved: _lib.Saved
    tensors: tuple
    saved_ws: torch.Tensor
    shape: _lib.Shape
    dtype: torch.dtype
    dt_bias: torch.Tensor | None = None

    def intermediates(self):
        """Views into the saved workspace: cs [b, H, K, Q] float32 and
        hin [b, K, H, P, N] (entry state of each chunk, storage dtype), with
        K = ceil(seqlen / chunk) (a shorter last chunk is zero-padded)."""
        s = self.shape
        K = -(-s.seqlen // s.chunk)
        ncs = s.batch * s.nheads * K * s.chunk
        cs = self.saved_ws[: ncs * 4].view(torch.float32).view(s.batch, s.nheads, K, s.chunk)
        off = (ncs * 4 + _ALIGN - 1) // _ALIGN * _ALIGN
        esz = 2 if self.dtype == torch.bfloat16 else 4
        nst = s.batch * K * s.nheads * s.headdim * s.dstate
        hin = self.saved_ws[off: off + nst * esz].view(self.dtype).view(s.batch, K, s.nheads, s.headdim, s.dstate)
        return cs, hin


def shape_of(x, B, chunk, dtype_code, flags=0) -> _lib.Shape:
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return _lib.make_shape(b, L, H, P, N, G, chunk, dtype_code, flags)


def _step_dtype(x_dtype):
    """dtype of dt, y and the gradients: x's, or bfloat16 when x, B, C are FP8."""
    return torch.bfloat16 if x_dtype == torch.float8_e4m3fn else x_dtype


def _validate(x, dt, A, B, C, D):
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be bfloat16, float32 or float8_e4m3fn, got {x.dtype}")
    for name, t, want in (("dt", dt, _step_dtype(x.dtype)), ("B", B, x.dtype), ("C", C, x.dtype)):
        if t.dtype != want:
            raise TypeError(f"{name} must have dtype {want}, got {t.dtype}")
    for name, t in (("A", A), ("D", D)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    for name, t in (("x", x), ("dt", dt), ("A", A), ("B", B), ("C", C), ("D", D)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    b, L, H, P = x.shape
    if dt.shape != (b, L, H) or A.shape != (H,) or D.shape != (H,):
        raise ValueError("shape mismatch among x, dt, A, D")
    if B.shape[:2] != (b, L) or C.shape != B.shape:
        raise ValueError("shape mismatch among x, B, C")


def _check_state(t, shape, name):
    if t is None:
        return
    want = (shape.batch, shape.nheads, shape.headdim, shape.dstate)
    if t.dtype != torch.float32 or tuple(t.shape) != want or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor of shape {want}")


def fwd(x, dt, A, B, C, D, chunk: int, *, initial_state: torch.Tensor | None = None,
        dt_softplus: bool = False, dt_bias: torch.Tensor | None = None, stream=None,
        probe: _lib.Probe | None = None, out: torch.Tensor | None = None, scratch: torch.Tensor | None = None,
        want_final_state: bool = True):
    """Forward pass from initial_state (zero if None).  With dt_softplus, dt is
    the raw step and the scan uses softplus(dt + dt_bias) (dt_bias [H] float32,
    zero if None).  Returns (y, final_state or None, Context)."""
    lib = _lib.load()
    _validate(x, dt, A, B, C, D)
    if dt_bias is not None:
        if not dt_softplus:
            raise ValueError("dt_bias is only used with dt_softplus=True")
        if dt_bias.dtype != torch.float32 or tuple(dt_bias.shape) != (x.shape[2],) or not dt_bias.is_cuda:
            raise ValueError("dt_bias must be a float32 GPU tensor of shape [nheads]")
    shape = shape_of(x, B, chunk, _DTYPES[x.dtype], _lib.SSD_DT_SOFTPLUS if dt_softplus else 0)
    _check_state(initial_state, shape, "initial_state")
    _check(lib.ssd_check_shape(ctypes.byref(shape)), "ssd_fwd")
    dev = x.device
    saved_bytes = lib.ssd_saved_bytes(ctypes.byref(shape))
    scratch_bytes = lib.ssd_fwd_scratch_bytes(ctypes.byref(shape))
    y = out if out is not None else torch.empty(x.shape, dtype=_step_dtype(x.dtype), device=x.device)
    fs = torch.empty((shape.batch, shape.nheads, shape.headdim, shape.dstate), dtype=torch.float32,
                     device=dev) if want_final_state else None
    saved_ws = torch.empty(saved_bytes, dtype=torch.uint8, device=dev)
    if scratch is None or scratch.numel() < scratch_bytes:
        scratch = torch.empty(scratch_bytes, dtype=torch.uint8, device=dev)
    saved = _lib.Saved()
    code = lib.ssd_fwd(ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                       _ptr(dt_bias) if dt_bias is not None else None,
                       _ptr(initial_state) if initial_state is not None else None, _ptr(y), _ptr(fs) if fs is not None else None, _ptr(saved_ws), saved_bytes,
                       ctypes.byref(saved), _ptr(scratch), scratch.numel(), _stream_handle(stream),
                       ctypes.byref(probe) if probe is not None else None)
    _check(code, "ssd_fwd")
    ctx = Context(saved, (x, dt, A, B, C, D), saved_ws, shape, _step_dtype(x.dtype), dt_bias)
    return y, fs, ctx


def bwd(dy, ctx: Context, *, dfinal_state: torch.Tensor | None = None, want_dinitial_state: bool = False,
        stream=None, probe: _lib.Probe | None = None, scratch: torch.Tensor | None = None):
    """Backward pass: gradients of sum(dy * y) + sum(dfinal_state * final_state)
    (dfinal_state None means zero).  Returns a dict of tensors, with
    dinitial_state when want_dinitial_state is set and, for a forward with
    dt_softplus, ddt_bias (ddt is then the gradient of the raw step)."""
    lib = _lib.load()
    x, dt, A, B, C, D = ctx.tensors
    gdt = _step_dtype(x.dtype)   # dy and the gradients: bfloat16 when x, B, C are FP8
    if dy.dtype != gdt or dy.shape != x.shape or not dy.is_contiguous() or not dy.is_cuda:
        raise ValueError(f"dy must be a contiguous GPU tensor with x's shape and dtype {gdt}")
    _check_state(dfinal_state, ctx.shape, "dfinal_state")
    scratch_bytes = lib.ssd_bwd_scratch_bytes(ctypes.byref(ctx.shape))
    if scratch is None or scratch.numel() < scratch_bytes:
        scratch = torch.empty(scratch_bytes, dtype=torch.uint8, device=x.device)
    dx = torch.empty(x.shape, dtype=gdt, device=x.device)
    ddt = torch.empty_like(dt)
    dB = torch.empty(B.shape, dtype=gdt, device=x.device)
    dC = torch.empty(C.shape, dtype=gdt, device=x.device)
    dA = torch.empty_like(A)
    dD = torch.empty_like(D)
    s = ctx.shape
    ds0 = torch.empty((s.batch, s.nheads, s.headdim, s.dstate), dtype=torch.float32,
                      device=x.device) if want_dinitial_state else None
    softplus = bool(s.flags & _lib.SSD_DT_SOFTPLUS)
    dbias = torch.empty_like(A) if softplus else None
    code = lib.ssd_bwd(ctypes.byref(ctx.saved), _ptr(dy), _ptr(dfinal_state) if dfinal_state is not None else None,
                       _ptr(dx), _ptr(ddt), _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dD),
                       _ptr(dbias) if dbias is not None else None,
                       _ptr(ds0) if ds0 is not None else None, _ptr(scratch), scratch.numel(),
                       _stream_handle(stream), ctypes.byref(probe) if probe is not None else None)
    _check(code, "ssd_bwd")
    g = dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD)
    if ds0 is not None:
        g["dinitial_state"] = ds0
    if dbias is not None:
        g["ddt_bias"] = dbias
    return g


def _conv_shape(x, w, silu):
    b, L, C = x.shape
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    if w.dtype != torch.float32 or w.dim() != 2 or w.shape[0] != C:
        raise ValueError("w must be float32 [channels, width]")
    return _lib.ConvShape(b, L, C, w.shape[1], _DTYPES[x.dtype], 1 if silu else 0, 0)


def _check_conv_tensors(shape, x, w, bias, x_prev):
    for name, t in (("x", x), ("w", w), ("bias", bias), ("x_prev", x_prev)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if bias is not None and (bias.dtype != torch.float32 or tuple(bias.shape) != (shape.channels,)):
        raise ValueError("bias must be float32 [channels]")
    if x_prev is not None and (x_prev.dtype != x.dtype
                               or tuple(x_prev.shape) != (shape.batch, shape.width - 1, shape.channels)):
        raise ValueError("x_prev must have x's dtype and shape [batch, width - 1, channels]")


def conv1d_fwd(x, w, bias=None, x_prev=None, silu=True, *, stream=None):
    """Causal depthwise conv1d: y[b,t,c] = act(bias[c] + sum_k w[c,k] x[b,t-(W-1)+k,c]).
    x [b, L, C] (bf16 or fp32), w [C, W] fp32, bias [C] fp32, x_prev [b, W-1, C] (rows before t = 0)."""
    lib = _lib.load()
    shape = _conv_shape(x, w, silu)
    _check_conv_tensors(shape, x, w, bias, x_prev)
    _check(lib.ssd_conv1d_check_shape(ctypes.byref(shape)), "ssd_conv1d_fwd")
    y = torch.empty_like(x)
    code = lib.ssd_conv1d_fwd(ctypes.byref(shape), _ptr(x), _ptr(w), _ptr(bias) if bias is not None else None,
                              _ptr(x_prev) if x_prev is not None else None, _ptr(y), _stream_handle(stream))
    _check(code, "ssd_conv1d_fwd")
    return y


def conv1d_bwd(x, w, dy, bias=None, x_prev=None, silu=True, *, want_dx_prev=False, stream=None):
    """Gradients of <dy, conv1d_fwd(...)>: dict dx, dw, dbias (if bias given), dx_prev (on request)."""
    lib = _lib.load()
    shape = _conv_shape(x, w, silu)
    _check_conv_tensors(shape, x, w, bias, x_prev)
    if dy.shape != x.shape or dy.dtype != x.dtype or not dy.is_contiguous() or not dy.is_cuda:
        raise ValueError("dy must be a contiguous GPU tensor with x's shape and dtype")
    _check(lib.ssd_conv1d_check_shape(ctypes.byref(shape)), "ssd_conv1d_bwd")
    nbytes = lib.ssd_conv1d_bwd_scratch_bytes(ctypes.byref(shape))
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    dx = torch.empty_like(x)
    dw = torch.empty_like(w)
    dbias = torch.empty_like(bias) if bias is not None else None
    dprev = torch.empty((shape.batch, shape.width - 1, shape.channels), dtype=x.dtype,
                        device=x.device) if want_dx_prev else None
    code = lib.ssd_conv1d_bwd(ctypes.byref(shape), _ptr(x), _ptr(w), _ptr(bias) if bias is not None else None,
                              _ptr(x_prev) if x_prev is not None else None, _ptr(dy), _ptr(dx), _ptr(dw),
                              _ptr(dbias) if dbias is not None else None, _ptr(dprev) if dprev is not None else None,
                              _ptr(scratch), nbytes, _stream_handle(stream))
    _check(code, "ssd_conv1d_bwd")
    g = dict(dx=dx, dw=dw)
    if dbias is not None:
        g["dbias"] = dbias
    if dprev is not None:
        g["dx_prev"] = dprev
    return g


def to_device(inp, device="cuda"):
    """Upload a seeded numpy draw (inputs.Inputs) as torch tensors of its storage dtype."""
    import numpy as np

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        if a.dtype == np.uint8:
            return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return dict(x=t(inp.x), dt=t(inp.dt), A=t(inp.A), B=t(inp.B), C=t(inp.C), D=t(inp.D), dy=t(inp.dy),
                dt_raw=t(inp.dt_raw), dt_bias=t(inp.dt_bias))
