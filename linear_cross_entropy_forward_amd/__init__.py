"""Fused linear cross-entropy (Cut Cross-Entropy) for AMD MI355X (gfx950).

Thin ctypes binding over libcce.so (C ABI declared in include/cce.h).  The
binding only marshals arguments: every step of the forward and backward runs
in the library's HIP kernels, on the caller's current torch stream.  PyTorch
provides device memory and streams.

    loss = linear_cross_entropy(e, c, targets)             # [..., D], [V, D], [...]
    loss, lse, n_valid, state = forward(e, c, targets)     # raw C-ABI calls
    dE, dC = backward(e, c, targets, lse, grad, state)

There is no fallback: without the built library (or without a GPU) every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["forward", "backward", "read_stats", "state_size", "workspace_size", "linear_cross_entropy", "cce_loss",
           "tile_shape", "lib", "CCEError", "library_path"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libcce.so")

CCE_OK = 0
_REDUCTIONS = {"none": 0, "sum": 1, "mean": 2}
_ACCUM = {"deterministic": 0, "atomic": 1}
_GRAD_DTYPE = {"float32": 0, "operand": 1}


class CCEError(RuntimeError):
    pass


class _Stats(ctypes.Structure):
    _fields_ = [("n_valid", ctypes.c_int64), ("bad_targets", ctypes.c_int64),
                ("tiles_total", ctypes.c_int64), ("tiles_kept", ctypes.c_int64),
                ("filter_rows", ctypes.c_int64), ("filter_vocab", ctypes.c_int64),
                ("blocks_total", ctypes.c_int64), ("blocks_kept", ctypes.c_int64),
                ("block_rows", ctypes.c_int64), ("block_vocab", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcce.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise CCEError(f"{library_path} is missing: build it with "
                       f"`python -m linear_cross_entropy_forward_amd.build`")
    L = ctypes.CDLL(library_path)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.cce_state_size.restype = sz
    L.cce_state_size.argtypes = [i64, i64, i64, i32]
    L.cce_workspace_size.restype = sz
    L.cce_workspace_size.argtypes = [i64, i64, i64, i32, i64]
    L.cce_vocab_chunk.restype = i64
    L.cce_vocab_chunk.argtypes = [i64, i64, i64, i32, i64]
    L.cce_forward.restype = i32
    L.cce_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i64, i32, f32, f32, f32, vp, vp, vp, vp, sz,
                              vp]
    L.cce_forward_noalloc.restype = i32
    L.cce_forward_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i64, i32, f32, f32, f32, vp, vp, vp, vp]
    L.cce_backward.restype = i32
    L.cce_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i64, i32, f32, f32, f32, vp, vp, i32, i32, i64,
                               i32, vp, vp, vp, vp, sz, vp, sz, vp]
    L.cce_read_stats.restype = i32
    L.cce_read_stats.argtypes = [vp, sz, i64, i64, vp, ctypes.POINTER(_Stats)]
    L.cce_read_keep_map.restype = i32
    L.cce_read_keep_map.argtypes = [vp, sz, i64, i64, i64, i32, i64, vp, vp]
    L.cce_read_block_map.restype = i32
    L.cce_read_block_map.argtypes = [vp, sz, i64, i64, i64, i32, i64, vp, vp]
    L.cce_status_string.restype = ctypes.c_char_p
    L.cce_status_string.argtypes = [i32]
    L.cce_tile_shape.restype = None
    L.cce_tile_shape.argtypes = [ctypes.POINTER(i32)] * 3
    L.cce_profile_start.restype = i32
    L.cce_profile_start.argtypes = [i32, i32]
    L.cce_profile_stop.restype = i32
    L.cce_profile_stop.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
    L.cce_kernel_name.restype = ctypes.c_char_p
    L.cce_kernel_name.argtypes = [i32]
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != CCE_OK:
        msg = lib().cce_status_string(status).decode()
        raise CCEError(f"{what}: {msg} ({status})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return 0
    if t.dtype == torch.float32:
        return 1
    raise CCEError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def tile_shape() -> tuple[int, int, int]:
    """(token rows, vocab entries) of a gradient tile and the forward partial width."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib().cce_tile_shape(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def state_size(N: int, D: int, V: int, dtype: torch.dtype = torch.bfloat16) -> int:
    """Bytes of the forward state (cce_state_size): what the backward needs
    from the forward."""
    code = 0 if dtype == torch.bfloat16 else 1
    n = lib().cce_state_size(N, D, V, code)
    if n == 0:
        raise CCEError("invalid sizes for cce_state_size")
    return n


def workspace_size(N: int, D: int, V: int, dtype: torch.dtype = torch.bfloat16, vocab_chunk: int = 0) -> int:
    """Bytes of the backward's scratch workspace (cce_workspace_size)."""
    code = 0 if dtype == torch.bfloat16 else 1
    n = lib().cce_workspace_size(N, D, V, code, vocab_chunk)
    if n == 0:
        raise CCEError("invalid sizes for cce_workspace_size")
    return n


def vocab_chunk(N: int, D: int, V: int, dtype: torch.dtype = torch.bfloat16, vocab_chunk: int = 0) -> int:
    """Vocabulary entries per backward chunk (cce_vocab_chunk)."""
    code = 0 if dtype == torch.bfloat16 else 1
    n = lib().cce_vocab_chunk(N, D, V, code, vocab_chunk)
    if n == 0:
        raise CCEError("invalid sizes for cce_vocab_chunk")
    return n


def _validate(e: torch.Tensor, c: torch.Tensor, targets: torch.Tensor) -> None:
    if not (e.is_cuda and c.is_cuda and targets.is_cuda):
        raise CCEError("e, c and targets must be device tensors")
    if e.dim() != 2 or c.dim() != 2 or e.shape[1] != c.shape[1]:
        raise CCEError(f"expected e [N, D] and c [V, D], got {tuple(e.shape)} and {tuple(c.shape)}")
    if e.dtype != c.dtype:
        raise CCEError("e and c must share a dtype")
    if targets.dtype != torch.int64 or targets.shape != (e.shape[0],):
        raise CCEError("targets must be int64 [N]")
    if not (e.is_contiguous() and c.is_contiguous() and targets.is_contiguous()):
        raise CCEError("e, c and targets must be contiguous")


def _validate_bias(bias, c):
    if bias is None:
        return
    if not bias.is_cuda or bias.dtype != c.dtype or bias.dim() != 1 or bias.shape[0] != c.shape[0] \
            or not bias.is_contiguous():
        raise CCEError(f"bias must be a contiguous device tensor [{c.shape[0]}] of dtype {c.dtype}")


def forward(e: torch.Tensor, c: torch.Tensor, targets: torch.Tensor, ignore_index: int = -100,
            reduction: str = "mean", softcap: float = 0.0, state: torch.Tensor | None = None,
            bias: torch.Tensor | None = None, label_smoothing: float = 0.0, z_loss: float = 0.0):
    """cce_forward.  Returns (loss, lse, n_valid, state); loss is [N] for
    reduction='none', else a 0-dim tensor.  `state` (uint8, device; the
    per-block partials and counters, O(N + N V / 128) floats) is allocated if
    not given and must be passed unchanged to backward().  `bias` [V] (the
    classifier's dtype) is optional; label_smoothing (eps in [0, 1]) and
    z_loss (lam >= 0) add the soft-target and lam * LSE^2 terms; softcap = s > 0
    replaces the logits by s * tanh(z / s) (not with label smoothing)."""
    _validate(e, c, targets)
    _validate_bias(bias, c)
    N, D = e.shape
    V = c.shape[0]
    dev = e.device
    if state is None:
        state = torch.empty(state_size(N, D, V, e.dtype), dtype=torch.uint8, device=dev)
    red = _REDUCTIONS[reduction]
    loss = torch.empty(N if red == 0 else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib().cce_forward(_ptr(e), _ptr(c), _ptr(bias) if bias is not None else None, _ptr(targets), N, D, V,
                             _dtype_code(e), ignore_index, red, softcap, label_smoothing, z_loss,
                             _ptr(loss), _ptr(lse), _ptr(n_valid), _ptr(state), state.numel(), _stream()),
           "cce_forward")
    return (loss if red == 0 else loss[0]), lse, n_valid, state


def backward(e: torch.Tensor, c: torch.Tensor, targets: torch.Tensor, lse: torch.Tensor,
             grad_loss: torch.Tensor, state: torch.Tensor, ignore_index: int = -100, reduction: str = "mean",
             filter: bool = True, accum: str = "deterministic", softcap: float = 0.0, vocab_chunk: int = 0,
             dE: torch.Tensor | None = None, dC: torch.Tensor | None = None, bias: torch.Tensor | None = None,
             want_dbias: bool = False, label_smoothing: float = 0.0, z_loss: float = 0.0,
             grad_dtype: str = "float32", want_dE: bool = True, want_dC: bool = True,
             ws: torch.Tensor | None = None):
    """cce_backward.  `state` is the forward's.  `ws` (uint8, device) is the
    call's scratch workspace: allocated here when not given (and released
    with the call's last reference).  grad_loss is float32 [N] ('none') or [1]/0-dim.  Returns
    (dE [N, D], dC [V, D]), plus float32 db [V] when want_dbias; dE and dC are
    float32, or with grad_dtype='operand' in e's dtype (written by the kernels,
    accumulated in fp32).  want_dE / want_dC = False leaves that gradient out
    (None; its contraction does not run).  bias, label_smoothing, z_loss and
    softcap must be those of the forward that filled the state."""
    _validate(e, c, targets)
    _validate_bias(bias, c)
    N, D = e.shape
    V = c.shape[0]
    dev = e.device
    g = grad_loss.reshape(-1).to(torch.float32).contiguous()
    gdt = torch.float32 if grad_dtype == "float32" else e.dtype
    if dE is None and want_dE:
        dE = torch.empty((N, D), dtype=gdt, device=dev)
    if dC is None and want_dC:
        dC = torch.empty((V, D), dtype=gdt, device=dev)
    for x in (dE, dC):
        if x is not None and (x.dtype != gdt or not x.is_contiguous()):
            raise CCEError(f"dE and dC must be contiguous {gdt} tensors")
    db = torch.empty(V, dtype=torch.float32, device=dev) if want_dbias else None
    if ws is None:
        ws = torch.empty(workspace_size(N, D, V, e.dtype, vocab_chunk), dtype=torch.uint8, device=dev)
    _check(lib().cce_backward(_ptr(e), _ptr(c), _ptr(bias) if bias is not None else None, _ptr(targets), N, D, V,
                              _dtype_code(e), ignore_index, _REDUCTIONS[reduction], softcap, label_smoothing,
                              z_loss, _ptr(lse), _ptr(g),
                              int(bool(filter)), _ACCUM[accum], vocab_chunk, _GRAD_DTYPE[grad_dtype],
                              _ptr(dE) if dE is not None else None, _ptr(dC) if dC is not None else None,
                              _ptr(db) if db is not None else None, _ptr(state), state.numel(), _ptr(ws),
                              ws.numel(), _stream()),
           "cce_backward")
    return (dE, dC, db) if want_dbias else (dE, dC)


def read_stats(state: torch.Tensor, N: int, V: int) -> dict:
    """Counters of the last forward/backward on `state` (synchronises the stream)."""
    s = _Stats()
    _check(lib().cce_read_stats(_ptr(state), state.numel(), N, V, _stream(), ctypes.byref(s)), "cce_read_stats")
    return {k: getattr(s, k) for k, _ in _Stats._fields_}


def read_keep_map(ws: torch.Tensor, N: int, D: int, V: int, dtype: torch.dtype = torch.bfloat16,
                  vocab_chunk: int = 0):
    """Tile keep map [ceil(N/256), ceil(V/256)] (numpy bool) of the last
    backward that used the workspace `ws` (synchronises the stream)."""
    import numpy as np
    nb, nvb = -(-N // 256), -(-V // 256)
    out = np.zeros((nb, nvb), dtype=np.uint8)
    code = 0 if dtype == torch.bfloat16 else 1
    _check(lib().cce_read_keep_map(_ptr(ws), ws.numel(), N, D, V, code, vocab_chunk,
                                   out.ctypes.data_as(ctypes.c_void_p), _stream()), "cce_read_keep_map")
    return out.astype(bool)


def read_block_map(ws: torch.Tensor, N: int, D: int, V: int, dtype: torch.dtype = torch.bfloat16,
                   vocab_chunk: int = 0):
    """32x32 block keep map [ceil(N/32), ceil(V/32)] (numpy bool) of the last
    backward that used the workspace `ws` (synchronises the stream)."""
    import numpy as np
    out = np.zeros((-(-N // 32), -(-V // 32)), dtype=np.uint8)
    code = 0 if dtype == torch.bfloat16 else 1
    _check(lib().cce_read_block_map(_ptr(ws), ws.numel(), N, D, V, code, vocab_chunk,
                                    out.ctypes.data_as(ctypes.c_void_p), _stream()), "cce_read_block_map")
    return out.astype(bool)


class _CCEFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, e, c, bias, targets, reduction, ignore_index, filter, accum, label_smoothing, z_loss,
                softcap):
        loss, lse, _, state = forward(e, c, targets, ignore_index=ignore_index, reduction=reduction, bias=bias,
                                      label_smoothing=label_smoothing, z_loss=z_loss, softcap=softcap)
        # only the forward state (partials and counters) is kept until the
        # backward; the backward's scratch is allocated there
        ctx.save_for_backward(e, c, bias, targets, lse, state)
        ctx.cfg = (reduction, ignore_index, filter, accum, label_smoothing, z_loss, softcap)
        return loss

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, grad):
        # first-order only: the kernels' gradients carry no graph of their own
        e, c, bias, targets, lse, state = ctx.saved_tensors
        reduction, ignore_index, filter, accum, label_smoothing, z_loss, softcap = ctx.cfg
        want_db = bias is not None and ctx.needs_input_grad[2]
        if not (ctx.needs_input_grad[0] or ctx.needs_input_grad[1] or want_db):
            return None, None, None, None, None, None, None, None, None, None, None
        # gradients in the inputs' dtype, written so by the kernels; a frozen
        # input's gradient is not formed
        out = backward(e, c, targets, lse, grad, state, ignore_index=ignore_index, reduction=reduction,
                       filter=filter, accum=accum, bias=bias, want_dbias=want_db,
                       label_smoothing=label_smoothing, z_loss=z_loss, softcap=softcap, grad_dtype="operand",
                       want_dE=ctx.needs_input_grad[0], want_dC=ctx.needs_input_grad[1])
        dE, dC = out[0], out[1]
        db = out[2].to(bias.dtype) if want_db else None
        return dE, dC, db, None, None, None, None, None, None, None, None


def cce_loss(e: torch.Tensor, c: torch.Tensor, targets: torch.Tensor, reduction: str = "mean",
             ignore_index: int = -100, filter: bool = True, accum: str = "deterministic",
             bias: torch.Tensor | None = None, label_smoothing: float = 0.0, z_loss: float = 0.0,
             softcap: float = 0.0) -> torch.Tensor:
    """Flat form: e [N, D], c [V, D], targets [N], optional bias [V]."""
    return _CCEFunction.apply(e.contiguous(), c.contiguous(), None if bias is None else bias.contiguous(),
                              targets.contiguous().to(torch.int64), reduction, ignore_index, filter, accum,
                              float(label_smoothing), float(z_loss), float(softcap))


def linear_cross_entropy(e: torch.Tensor, c: torch.Tensor, targets: torch.Tensor, bias=None,
                         reduction: str = "mean", ignore_index: int = -100, filter: bool = True,
                         accum: str = "deterministic", label_smoothing: float = 0.0,
                         z_loss: float = 0.0, softcap: float = 0.0) -> torch.Tensor:
    """Cross-entropy of softmax(e @ c.T + bias) against targets without forming
    the logits.  e [..., D], c [V, D], targets [...], bias [V] or None;
    'none' returns a tensor shaped like targets.  label_smoothing spreads eps
    over all V classes; z_loss adds z_loss * LSE^2 per row; softcap = s > 0
    soft-caps the logits to s * tanh(z / s)."""
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(_REDUCTIONS)}")
    shape = targets.shape
    D = e.shape[-1]
    out = cce_loss(e.reshape(-1, D), c, targets.reshape(-1), reduction, ignore_index, filter, accum, bias=bias,
                   label_smoothing=label_smoothing, z_loss=z_loss, softcap=softcap)
    return out.reshape(shape) if reduction == "none" else out
