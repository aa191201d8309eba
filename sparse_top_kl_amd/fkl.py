"""ctypes binding of libfkl (include/fkl.h), plus an autograd wrapper.

Argument marshalling only: tensors become device pointers, torch's current
HIP stream is passed through, and the library's status codes become
exceptions. Every step of the loss runs in libfkl's HIP kernels; there is no
CPU or PyTorch fallback. If the library is not built this module raises.

Functions with the ``fkl_`` prefix mirror the C entry points one to one;
``fused_chunked_kl`` is the user-facing loss with autograd.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FKL_LIBRARY") or os.path.join(HERE, "libfkl.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "fkl.h")


def _header_constants() -> dict:
    consts = {}
    with open(HEADER_PATH) as f:
        for m in re.finditer(r"#define\s+(FKL_\w+)\s+(\d+)u?", f.read()):
            consts[m.group(1)] = int(m.group(2))
    return consts


_C = _header_constants()
FKL_OK = _C["FKL_OK"]
FKL_E_ARG = _C["FKL_E_ARG"]
FKL_E_UNSUPPORTED = _C["FKL_E_UNSUPPORTED"]
FKL_E_WORKSPACE = _C["FKL_E_WORKSPACE"]
FKL_E_HIP = _C["FKL_E_HIP"]
FKL_E_INDEX = _C["FKL_E_INDEX"]
FKL_F32 = _C["FKL_F32"]
FKL_BF16 = _C["FKL_BF16"]
FKL_FLAG_ACCUMULATE_GRAD_W = _C["FKL_FLAG_ACCUMULATE_GRAD_W"]
FKL_FLAG_VALIDATE_IDX = _C["FKL_FLAG_VALIDATE_IDX"]


class FklError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libfkl status {status}: {message}")
        self.status = status


_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

class LossOptions(ctypes.Structure):
    """Mirror of fkl_loss_options (include/fkl.h)."""
    _fields_ = [("row_weight", ctypes.c_void_p), ("labels", ctypes.c_void_p),
                ("alpha", ctypes.c_float), ("lse1", ctypes.c_void_p),
                ("teacher_lse", ctypes.c_void_p)]


_opt = ctypes.POINTER(LossOptions)

_SIGNATURES = {
    "fkl_abi_version": (_i32, []),
    "fkl_status_string": (ctypes.c_char_p, [_i32]),
    "fkl_last_error": (ctypes.c_char_p, []),
    "fkl_workspace_size": (_i32, [_i64, _i64, _i64, _i32, _i64, _i32,
                                  ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "fkl_forward": (_i32, [_p, _p, _p, _p, _f32, _i64, _i64, _i64, _i64, _i32, _i32, _u32,
                           _p, _p, _p, _p, _p, _sz, _p]),
    "fkl_backward": (_i32, [_p, _p, _p, _p, _p, _p, _p, _f32, _i64, _i64, _i64, _i64, _i32,
                            _i32, _u32, _p, _p, _p, _sz, _p]),
    "fkl_keep_sizes": (_i32, [_i64, _i64, _i64, _i32, _i32,
                              ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "fkl_forward_keep": (_i32, [_p, _p, _p, _p, _f32, _i64, _i64, _i64, _i64, _i32, _i32, _u32,
                                _p, _p, _p, _p, _p, _sz, _p, _sz, _p]),
    "fkl_backward_keep": (_i32, [_p, _p, _p, _p, _p, _p, _p, _f32, _i64, _i64, _i64, _i32,
                                 _i32, _u32, _p, _sz, _p, _p, _p, _sz, _p]),
    "fkl_topk_workspace_size": (_i32, [_i64, _i64, _i64, _i32, _i64, _i32,
                                       ctypes.POINTER(_sz)]),
    "fkl_teacher_topk": (_i32, [_p, _p, _i64, _i64, _i64, _i32, _i64, _i32, _u32, _p, _p, _p,
                                _sz, _p]),
    "fkl_forward_ex": (_i32, [_p, _p, _p, _p, _f32, _i64, _i64, _i64, _i64, _i32, _i32, _u32,
                              _opt, _p, _p, _p, _p, _p, _sz, _p]),
    "fkl_backward_ex": (_i32, [_p, _p, _p, _p, _p, _p, _p, _f32, _i64, _i64, _i64, _i64, _i32,
                               _i32, _u32, _opt, _p, _p, _p, _sz, _p]),
    "fkl_forward_keep_ex": (_i32, [_p, _p, _p, _p, _f32, _i64, _i64, _i64, _i64, _i32, _i32,
                                   _u32, _opt, _p, _p, _p, _p, _p, _sz, _p, _sz, _p]),
    "fkl_backward_keep_ex": (_i32, [_p, _p, _p, _p, _p, _p, _p, _f32, _i64, _i64, _i64, _i32,
                                    _i32, _u32, _opt, _p, _sz, _p, _p, _p, _sz, _p]),
    "fkl_teacher_topk_ex": (_i32, [_p, _p, _i64, _i64, _i64, _i32, _i64, _i32, _u32, _f32, _p,
                                   _p, _p, _p, _sz, _p]),
    "fkl_renorm_workspace_size": (_i32, [_i64, _i64, _i64, _i32, _i32, ctypes.POINTER(_sz),
                                         ctypes.POINTER(_sz)]),
    "fkl_renorm_forward": (_i32, [_p, _p, _p, _p, _f32, _i64, _i64, _i64, _i32, _i32, _u32, _p,
                                  _p, _p, _p, _p, _sz, _p]),
    "fkl_renorm_backward": (_i32, [_p, _p, _p, _p, _p, _p, _f32, _i64, _i64, _i64, _i32, _i32,
                                   _u32, _p, _p, _p, _p, _sz, _p]),
    "fkl_forward_noalloc": (_i32, [_p, _p, _p, _p, _f32, _i64, _i64, _i64, _i64, _i32, _i32,
                                   _u32, _p, _p, _p, _p, _p]),
    "fkl_timing_enable": (_i32, [_i32]),
    "fkl_timing_reset": (_i32, []),
    "fkl_timing_read": (_i32, [_i32, ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double)]),
    "fkl_kernel_count": (_i32, []),
    "fkl_kernel_name": (ctypes.c_char_p, [_i32]),
}


def lib() -> ctypes.CDLL:
    """The loaded libfkl.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_top_kl_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != FKL_OK:
        raise FklError(status, f"{fkl_status_string(status)}: {fkl_last_error()}")


def fkl_abi_version() -> int:
    return lib().fkl_abi_version()


def fkl_status_string(status: int) -> str:
    return lib().fkl_status_string(status).decode()


def fkl_last_error() -> str:
    return lib().fkl_last_error().decode()


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return FKL_BF16
    if dt == torch.float32:
        return FKL_F32
    raise FklError(FKL_E_UNSUPPORTED, f"hidden/weight dtype {dt} (bf16 or fp32 only)")


def fkl_workspace_size(N, d, V, K, chunk, dtype) -> tuple[int, int]:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    f, b = _sz(0), _sz(0)
    _check(lib().fkl_workspace_size(N, d, V, K, chunk, code, ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _require(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise FklError(FKL_E_ARG, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise FklError(FKL_E_ARG, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise FklError(FKL_E_ARG, f"{name} must be {dtype}, got {t.dtype}")


@dataclass
class ForwardResult:
    loss: torch.Tensor       # [] fp32
    lse: torch.Tensor        # [N] fp32
    row_loss: torch.Tensor   # [N] fp32
    topk_z: torch.Tensor     # [N, K] fp32
    lse1: torch.Tensor | None = None   # [N] fp32, temperature-1 lse (with labels)


def _loss_options(N, row_weight, labels, alpha, lse1, teacher_lse=None):
    """(LossOptions, keep-alive tensors) for the *_ex entry points."""
    keep = []
    if row_weight is not None:
        row_weight = row_weight.reshape(-1).to(torch.float32).contiguous()
        _require(row_weight, "row_weight", torch.float32)
        if row_weight.numel() != N:
            raise FklError(FKL_E_ARG, "row_weight must have N entries")
        keep.append(row_weight)
    if labels is not None:
        labels = labels.reshape(-1).to(torch.int32).contiguous()
        _require(labels, "labels", torch.int32)
        if labels.numel() != N:
            raise FklError(FKL_E_ARG, "labels must have N entries")
        keep.append(labels)
    if lse1 is not None:
        _require(lse1, "lse1", torch.float32)
        if lse1.numel() != N:
            raise FklError(FKL_E_ARG, "lse1 must have N entries")
        keep.append(lse1)
    if teacher_lse is not None:
        teacher_lse = teacher_lse.reshape(-1).to(torch.float32).contiguous()
        _require(teacher_lse, "teacher_lse", torch.float32)
        if teacher_lse.numel() != N:
            raise FklError(FKL_E_ARG, "teacher_lse must have N entries")
        keep.append(teacher_lse)
    o = LossOptions(_ptr(row_weight), _ptr(labels), float(alpha), _ptr(lse1), _ptr(teacher_lse))
    return o, keep


def fkl_forward(hidden: torch.Tensor, weight: torch.Tensor, topk_idx: torch.Tensor,
                topk_logit: torch.Tensor, T: float, chunk: int, *, validate: bool = False,
                workspace: torch.Tensor | None = None) -> ForwardResult:
    """Forward pass on [N, d] hidden, [V, d] weight, [N, K] int32 ids and fp32 logits."""
    N, d = hidden.shape
    V, K = weight.shape[0], topk_idx.shape[1]
    code = dtype_code(hidden.dtype)
    for t, n, dt in ((hidden, "hidden", None), (weight, "weight", hidden.dtype),
                     (topk_idx, "topk_idx", torch.int32), (topk_logit, "topk_logit", torch.float32)):
        _require(t, n, dt)
    dev = hidden.device
    fw, _ = fkl_workspace_size(N, d, V, K, chunk, code)
    ws = workspace if workspace is not None else _workspace(fw, dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    row_loss = torch.empty(N, dtype=torch.float32, device=dev)
    topk_z = torch.empty(N, K, dtype=torch.float32, device=dev)
    flags = FKL_FLAG_VALIDATE_IDX if validate else 0
    _check(lib().fkl_forward(_ptr(hidden), _ptr(weight), _ptr(topk_idx), _ptr(topk_logit),
                             float(T), chunk, N, d, V, K, code, flags, _ptr(loss), _ptr(lse),
                             _ptr(row_loss), _ptr(topk_z), _ptr(ws), ws.numel(), _stream(dev)))
    return ForwardResult(loss, lse, row_loss, topk_z)


def fkl_forward_noalloc(hidden: torch.Tensor, weight: torch.Tensor, topk_idx: torch.Tensor,
                        topk_logit: torch.Tensor, T: float, chunk: int, *, out: ForwardResult,
                        validate: bool = False) -> ForwardResult:
    """fkl_forward on the library's static per-device scratch (no workspace,
    no allocation): the outputs are written into ``out`` (loss [] and lse [N]
    required; row_loss [N] and topk_z [N, K] may be None)."""
    N, d = hidden.shape
    V, K = weight.shape[0], topk_idx.shape[1]
    code = dtype_code(hidden.dtype)
    for t, n, dt in ((hidden, "hidden", None), (weight, "weight", hidden.dtype),
                     (topk_idx, "topk_idx", torch.int32), (topk_logit, "topk_logit", torch.float32),
                     (out.loss, "loss", torch.float32), (out.lse, "lse", torch.float32)):
        _require(t, n, dt)
    for t, n in ((out.row_loss, "row_loss"), (out.topk_z, "topk_z")):
        if t is not None:
            _require(t, n, torch.float32)
    flags = FKL_FLAG_VALIDATE_IDX if validate else 0
    _check(lib().fkl_forward_noalloc(_ptr(hidden), _ptr(weight), _ptr(topk_idx),
                                     _ptr(topk_logit), float(T), chunk, N, d, V, K, code, flags,
                                     _ptr(out.loss), _ptr(out.lse), _ptr(out.row_loss),
                                     _ptr(out.topk_z), _stream(hidden.device)))
    return out


def fkl_backward(hidden: torch.Tensor, weight: torch.Tensor, topk_idx: torch.Tensor,
                 topk_logit: torch.Tensor, lse: torch.Tensor, T: float, chunk: int, *,
                 topk_z: torch.Tensor | None = None, grad_loss: torch.Tensor | None = None,
                 grad_weight: torch.Tensor | None = None, accumulate: bool = False,
                 validate: bool = False, workspace: torch.Tensor | None = None):
    """Backward pass; returns (grad_hidden [N, d] in hidden's dtype, grad_weight [V, d] fp32)."""
    N, d = hidden.shape
    V, K = weight.shape[0], topk_idx.shape[1]
    code = dtype_code(hidden.dtype)
    for t, n, dt in ((hidden, "hidden", None), (weight, "weight", hidden.dtype),
                     (topk_idx, "topk_idx", torch.int32), (topk_logit, "topk_logit", torch.float32),
                     (lse, "lse", torch.float32)):
        _require(t, n, dt)
    if topk_z is not None:
        _require(topk_z, "topk_z", torch.float32)
    if grad_loss is not None:
        _require(grad_loss, "grad_loss", torch.float32)
    dev = hidden.device
    _, bw = fkl_workspace_size(N, d, V, K, chunk, code)
    ws = workspace if workspace is not None else _workspace(bw, dev)
    grad_hidden = torch.empty_like(hidden)
    if grad_weight is None:
        grad_weight = torch.empty(V, d, dtype=torch.float32, device=dev)
    else:
        _require(grad_weight, "grad_weight", torch.float32)
    flags = (FKL_FLAG_ACCUMULATE_GRAD_W if accumulate else 0) | \
        (FKL_FLAG_VALIDATE_IDX if validate else 0)
    _check(lib().fkl_backward(_ptr(hidden), _ptr(weight), _ptr(topk_idx), _ptr(topk_logit),
                              _ptr(lse), _ptr(topk_z), _ptr(grad_loss), float(T), chunk, N, d, V,
                              K, code, flags, _ptr(grad_hidden), _ptr(grad_weight), _ptr(ws),
                              ws.numel(), _stream(dev)))
    return grad_hidden, grad_weight


def keep_pitch(V: int) -> int:
    """Row pitch (elements) of the kept-logits buffer: V rounded up to 64."""
    return (V + 63) // 64 * 64


def fkl_keep_sizes(N, d, V, K, dtype) -> tuple[int, int]:
    """(kept-logits bytes, fkl_backward_keep workspace bytes)."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    z, b = _sz(0), _sz(0)
    _check(lib().fkl_keep_sizes(N, d, V, K, code, ctypes.byref(z), ctypes.byref(b)))
    return z.value, b.value


def fkl_forward_keep(hidden: torch.Tensor, weight: torch.Tensor, topk_idx: torch.Tensor,
                     topk_logit: torch.Tensor, T: float, chunk: int, *,
                     logits: torch.Tensor | None = None, validate: bool = False,
                     workspace: torch.Tensor | None = None):
    """Forward pass that also keeps the logits; returns (ForwardResult, logits
    [N, keep_pitch(V)] in hidden's dtype). The logits serve one fkl_backward_keep."""
    N, d = hidden.shape
    V, K = weight.shape[0], topk_idx.shape[1]
    code = dtype_code(hidden.dtype)
    for t, n, dt in ((hidden, "hidden", None), (weight, "weight", hidden.dtype),
                     (topk_idx, "topk_idx", torch.int32), (topk_logit, "topk_logit", torch.float32)):
        _require(t, n, dt)
    dev = hidden.device
    fw, _ = fkl_workspace_size(N, d, V, K, chunk, code)
    ws = workspace if workspace is not None else _workspace(fw, dev)
    if logits is None:
        logits = torch.empty(N, keep_pitch(V), dtype=hidden.dtype, device=dev)
    else:
        _require(logits, "logits", hidden.dtype)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    row_loss = torch.empty(N, dtype=torch.float32, device=dev)
    topk_z = torch.empty(N, K, dtype=torch.float32, device=dev)
    flags = FKL_FLAG_VALIDATE_IDX if validate else 0
    _check(lib().fkl_forward_keep(_ptr(hidden), _ptr(weight), _ptr(topk_idx), _ptr(topk_logit),
                                  float(T), chunk, N, d, V, K, code, flags, _ptr(loss), _ptr(lse),
                                  _ptr(row_loss), _ptr(topk_z), _ptr(logits),
                                  logits.numel() * logits.element_size(), _ptr(ws), ws.numel(),
                                  _stream(dev)))
    return ForwardResult(loss, lse, row_loss, topk_z), logits


def fkl_backward_keep(hidden: torch.Tensor, weight: torch.Tensor, topk_idx: torch.Tensor,
                      topk_logit: torch.Tensor, lse: torch.Tensor, T: float,
                      logits: torch.Tensor, *, topk_z: torch.Tensor | None = None,
                      grad_loss: torch.Tensor | None = None,
                      grad_weight: torch.Tensor | None = None, accumulate: bool = False,
                      validate: bool = False, workspace: torch.Tensor | None = None):
    """Backward from kept logits (which it overwrites with the logit gradient);
    returns (grad_hidden, grad_weight fp32) as fkl_backward."""
    N, d = hidden.shape
    V, K = weight.shape[0], topk_idx.shape[1]
    code = dtype_code(hidden.dtype)
    for t, n, dt in ((hidden, "hidden", None), (weight, "weight", hidden.dtype),
                     (topk_idx, "topk_idx", torch.int32), (topk_logit, "topk_logit", torch.float32),
                     (lse, "lse", torch.float32), (logits, "logits", hidden.dtype)):
        _require(t, n, dt)
    if topk_z is not None:
        _require(topk_z, "topk_z", torch.float32)
    if grad_loss is not None:
        _require(grad_loss, "grad_loss", torch.float32)
    dev = hidden.device
    _, bw = fkl_keep_sizes(N, d, V, K, code)
    ws = workspace if workspace is not None else _workspace(bw, dev)
    grad_hidden = torch.empty_like(hidden)
    if grad_weight is None:
        grad_weight = torch.empty(V, d, dtype=torch.float32, device=dev)
    else:
        _require(grad_weight, "grad_weight", torch.float32)
    flags = (FKL_FLAG_ACCUMULATE_GRAD_W if accumulate else 0) | \
        (FKL_FLAG_VALIDATE_IDX if validate else 0)
    _check(lib().fkl_backward_keep(_ptr(hidden), _ptr(weight), _ptr(topk_idx), _ptr(topk_logit),
                                   _ptr(lse), _ptr(topk_z), _ptr(grad_loss), float(T), N, d, V, K,
                                   code, flags, _ptr(logits),
                                   logits.numel() * logits.element_size(), _ptr(grad_hidden),
                                   _ptr(grad_weight), _ptr(ws), ws.numel(), _stream(dev)))
    return grad_hidden, grad_weight


def fkl_topk_workspace_size(N, d, V, K, chunk, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    b = _sz(0)
    _check(lib().fkl_topk_workspace_size(N, d, V, K, chunk, code, ctypes.byref(b)))
    return b.value


def fkl_teacher_topk(hidden: torch.Tensor, weight: torch.Tensor, K: int, chunk: int = 2048, *,
                     workspace: torch.Tensor | None = None):
    """Teacher top-K cache: per row of hidden [N, d] the K largest logits of
    hidden . weight^T (weight [V, d]), ordered by value with ties to the lower
    id. Returns (ids int32 [N, K], logits fp32 [N, K])."""
    N, d = hidden.shape
    V = weight.shape[0]
    code = dtype_code(hidden.dtype)
    _require(hidden, "hidden")
    _require(weight, "weight", hidden.dtype)
    dev = hidden.device
    nb = fkl_topk_workspace_size(N, d, V, K, chunk, code)
    ws = workspace if workspace is not None else _workspace(nb, dev)
    idx = torch.empty(N, K, dtype=torch.int32, device=dev)
    val = torch.empty(N, K, dtype=torch.float32, device=dev)
    _check(lib().fkl_teacher_topk(_ptr(hidden), _ptr(weight), N, d, V, K, chunk, code, 0,
                                  _ptr(idx), _ptr(val), _ptr(ws), ws.numel(), _stream(dev)))
    return idx, val


def fkl_forward_ex(hidden, weight, topk_idx, topk_logit, T: float, chunk: int, *,
                   row_weight=None, labels=None, alpha: float = 1.0, teacher_lse=None,
                   lse1=None, keep_logits=None, validate: bool = False, workspace=None):
    """fkl_forward (or with keep_logits, a [N, keep_pitch(V)] buffer or True,
    fkl_forward_keep) with loss options: per-row weights, hard labels (< 0:
    none) and the KL/cross-entropy mixing weight alpha. Returns a
    ForwardResult whose lse1 (the temperature-1 lse) is set when labels are
    given (the backward needs it) or an [N] fp32 lse1 buffer is passed, plus
    the kept logits in keep mode: (result, logits)."""
    N, d = hidden.shape
    V, K = weight.shape[0], topk_idx.shape[1]
    code = dtype_code(hidden.dtype)
    for t, n, dt in ((hidden, "hidden", None), (weight, "weight", hidden.dtype),
                     (topk_idx, "topk_idx", torch.int32), (topk_logit, "topk_logit", torch.float32)):
        _require(t, n, dt)
    dev = hidden.device
    fw, _ = fkl_workspace_size(N, d, V, K, chunk, code)
    ws = workspace if workspace is not None else _workspace(fw, dev)
    if lse1 is None and labels is not None:
        lse1 = torch.empty(N, dtype=torch.float32, device=dev)
    o, alive = _loss_options(N, row_weight, labels, alpha, lse1, teacher_lse)
    out = ForwardResult(torch.empty((), dtype=torch.float32, device=dev),
                        torch.empty(N, dtype=torch.float32, device=dev),
                        torch.empty(N, dtype=torch.float32, device=dev),
                        torch.empty(N, K, dtype=torch.float32, device=dev), lse1)
    flags = FKL_FLAG_VALIDATE_IDX if validate else 0
    common = (_ptr(hidden), _ptr(weight), _ptr(topk_idx), _ptr(topk_logit), float(T), chunk, N, d,
              V, K, code, flags, ctypes.byref(o), _ptr(out.loss), _ptr(out.lse),
              _ptr(out.row_loss), _ptr(out.topk_z))
    if keep_logits is None or keep_logits is False:
        _check(lib().fkl_forward_ex(*common, _ptr(ws), ws.numel(), _stream(dev)))
        return out
    z = keep_logits if isinstance(keep_logits, torch.Tensor) else \
        torch.empty(N, keep_pitch(V), dtype=hidden.dtype, device=dev)
    _require(z, "logits", hidden.dtype)
    _check(lib().fkl_forward_keep_ex(*common, _ptr(z), z.numel() * z.element_size(), _ptr(ws),
                                     ws.numel(), _stream(dev)))
    del alive
    return out, z


def fkl_backward_ex(hidden, weight, topk_idx, topk_logit, lse, T: float, chunk: int, *,
                    topk_z=None, grad_loss=None, row_weight=None, labels=None,
                    alpha: float = 1.0, lse1=None, teacher_lse=None, logits=None,
                    grad_weight=None, accumulate: bool = False, validate: bool = False,
                    workspace=None):
    """fkl_backward (or, given the kept logits, fkl_backward_keep) with loss
    options; lse1 is the forward's (required with labels when T != 1)."""
    N, d = hidden.shape
    V, K = weight.shape[0], topk_idx.shape[1]
    code = dtype_code(hidden.dtype)
    for t, n, dt in ((hidden, "hidden", None), (weight, "weight", hidden.dtype),
                     (topk_idx, "topk_idx", torch.int32), (topk_logit, "topk_logit", torch.float32),
                     (lse, "lse", torch.float32)):
        _require(t, n, dt)
    dev = hidden.device
    if logits is None:
        _, bw = fkl_workspace_size(N, d, V, K, chunk, code)
    else:
        _require(logits, "logits", hidden.dtype)
        _, bw = fkl_keep_sizes(N, d, V, K, code)
    ws = workspace if workspace is not None else _workspace(bw, dev)
    o, alive = _loss_options(N, row_weight, labels, alpha, lse1, teacher_lse)
    grad_hidden = torch.empty_like(hidden)
    if grad_weight is None:
        grad_weight = torch.empty(V, d, dtype=torch.float32, device=dev)
    flags = (FKL_FLAG_ACCUMULATE_GRAD_W if accumulate else 0) | \
        (FKL_FLAG_VALIDATE_IDX if validate else 0)
    head = (_ptr(hidden), _ptr(weight), _ptr(topk_idx), _ptr(topk_logit), _ptr(lse),
            _ptr(topk_z), _ptr(grad_loss), float(T))
    if logits is None:
        _check(lib().fkl_backward_ex(*head, chunk, N, d, V, K, code, flags, ctypes.byref(o),
                                     _ptr(grad_hidden), _ptr(grad_weight), _ptr(ws), ws.numel(),
                                     _stream(dev)))
    else:
        _check(lib().fkl_backward_keep_ex(*head, N, d, V, K, code, flags, ctypes.byref(o),
                                          _ptr(logits), logits.numel() * logits.element_size(),
                                          _ptr(grad_hidden), _ptr(grad_weight), _ptr(ws),
                                          ws.numel(), _stream(dev)))
    del alive
    return grad_hidden, grad_weight


def fkl_forward_keep_ex(hidden, weight, topk_idx, topk_logit, T, chunk, *, logits=None, **opts):
    """fkl_forward_keep with loss options; returns (ForwardResult, logits)."""
    return fkl_forward_ex(hidden, weight, topk_idx, topk_logit, T, chunk,
                          keep_logits=True if logits is None else logits, **opts)


def fkl_backward_keep_ex(hidden, weight, topk_idx, topk_logit, lse, T, logits, **opts):
    """fkl_backward_keep with loss options (the kept logits are consumed)."""
    return fkl_backward_ex(hidden, weight, topk_idx, topk_logit, lse, T, 1, logits=logits, **opts)


def fkl_teacher_topk_ex(hidden: torch.Tensor, weight: torch.Tensor, K: int, chunk: int = 2048,
                        *, T: float = 1.0, workspace: torch.Tensor | None = None):
    """fkl_teacher_topk plus the teacher's full-vocabulary log-sum-exp at T:
    returns (ids int32 [N, K], logits fp32 [N, K], teacher_lse fp32 [N])."""
    N, d = hidden.shape
    V = weight.shape[0]
    code = dtype_code(hidden.dtype)
    _require(hidden, "hidden")
    _require(weight, "weight", hidden.dtype)
    dev = hidden.device
    nb = fkl_topk_workspace_size(N, d, V, K, chunk, code)
    ws = workspace if workspace is not None else _workspace(nb, dev)
    idx = torch.empty(N, K, dtype=torch.int32, device=dev)
    val = torch.empty(N, K, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    _check(lib().fkl_teacher_topk_ex(_ptr(hidden), _ptr(weight), N, d, V, K, chunk, code, 0,
                                     float(T), _ptr(idx), _ptr(val), _ptr(lse), _ptr(ws),
                                     ws.numel(), _stream(dev)))
    return idx, val, lse


def fkl_renorm_workspace_size(N, d, V, K, dtype) -> tuple[int, int]:
    """(forward, backward) workspace bytes of the student-renormalised loss."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    f, b = _sz(0), _sz(0)
    _check(lib().fkl_renorm_workspace_size(N, d, V, K, code, ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


@dataclass
class RenormResult:
    loss: torch.Tensor      # [] fp32
    row_loss: torch.Tensor  # [N] fp32
    topk_z: torch.Tensor    # [N, K] fp32 student logits at the cached ids


def fkl_renorm_forward(hidden, weight, topk_idx, topk_logit, T: float, *,
                       row_weight: torch.Tensor | None = None, validate: bool = False,
                       workspace: torch.Tensor | None = None) -> RenormResult:
    """Student-renormalised top-K loss (both softmaxes over the K cached
    entries): fkl_renorm_forward of include/fkl.h."""
    N, d = hidden.shape
    V = weight.shape[0]
    K = topk_idx.shape[1]
    code = dtype_code(hidden.dtype)
    _require(hidden, "hidden")
    _require(weight, "weight", hidden.dtype)
    _require(topk_idx, "topk_idx", torch.int32)
    _require(topk_logit, "topk_logit", torch.float32)
    if row_weight is not None:
        _require(row_weight, "row_weight", torch.float32)
    dev = hidden.device
    fw, _ = fkl_renorm_workspace_size(N, d, V, K, code)
    ws = workspace if workspace is not None else _workspace(fw, dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    row_loss = torch.empty(N, dtype=torch.float32, device=dev)
    topk_z = torch.empty(N, K, dtype=torch.float32, device=dev)
    flags = FKL_FLAG_VALIDATE_IDX if validate else 0
    _check(lib().fkl_renorm_forward(_ptr(hidden), _ptr(weight), _ptr(topk_idx), _ptr(topk_logit),
                                    float(T), N, d, V, K, code, flags, _ptr(row_weight),
                                    _ptr(loss), _ptr(row_loss), _ptr(topk_z), _ptr(ws),
                                    ws.numel(), _stream(dev)))
    return RenormResult(loss, row_loss, topk_z)


def fkl_renorm_backward(hidden, weight, topk_idx, topk_logit, T: float, *,
                        topk_z: torch.Tensor | None = None,
                        grad_loss: torch.Tensor | None = None,
                        row_weight: torch.Tensor | None = None,
                        grad_weight: torch.Tensor | None = None, accumulate: bool = False,
                        validate: bool = False, workspace: torch.Tensor | None = None):
    """Gradients of the student-renormalised loss: (grad_hidden [N, d] in the
    input dtype, grad_weight [V, d] fp32)."""
    N, d = hidden.shape
    V = weight.shape[0]
    K = topk_idx.shape[1]
    code = dtype_code(hidden.dtype)
    _require(hidden, "hidden")
    _require(weight, "weight", hidden.dtype)
    _require(topk_idx, "topk_idx", torch.int32)
    _require(topk_logit, "topk_logit", torch.float32)
    for t, name in ((topk_z, "topk_z"), (grad_loss, "grad_loss"), (row_weight, "row_weight")):
        if t is not None:
            _require(t, name, torch.float32)
    dev = hidden.device
    _, bw = fkl_renorm_workspace_size(N, d, V, K, code)
    ws = workspace if workspace is not None else _workspace(bw, dev)
    gh = torch.empty(N, d, dtype=hidden.dtype, device=dev)
    gw = grad_weight if grad_weight is not None else torch.empty(V, d, dtype=torch.float32,
                                                                 device=dev)
    _require(gw, "grad_weight", torch.float32)
    flags = (FKL_FLAG_ACCUMULATE_GRAD_W if accumulate else 0) | (
        FKL_FLAG_VALIDATE_IDX if validate else 0)
    _check(lib().fkl_renorm_backward(_ptr(hidden), _ptr(weight), _ptr(topk_idx),
                                     _ptr(topk_logit), _ptr(topk_z), _ptr(grad_loss), float(T),
                                     N, d, V, K, code, flags, _ptr(row_weight), _ptr(gh), _ptr(gw),
                                     _ptr(ws), ws.numel(), _stream(dev)))
    return gh, gw


def fkl_timing_enable(on: bool) -> bool:
    """Turns per-kernel event timing on or off; returns the previous state."""
    return bool(lib().fkl_timing_enable(1 if on else 0))


def fkl_timing_reset() -> None:
    _check(lib().fkl_timing_reset())


def fkl_timing_read(kernel: int) -> tuple[int, float]:
    """(launches, total milliseconds) of one kernel since the last reset."""
    n, ms = _i64(0), ctypes.c_double(0.0)
    _check(lib().fkl_timing_read(kernel, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def fkl_kernel_count() -> int:
    return lib().fkl_kernel_count()


def fkl_kernel_name(kernel: int) -> str | None:
    r = lib().fkl_kernel_name(kernel)
    return None if r is None else r.decode()


def kernel_times() -> dict:
    """{kernel name: (launches, total ms)} for every kernel since the last reset."""
    out = {}
    for k in range(fkl_kernel_count()):
        n, ms = fkl_timing_read(k)
        if n:
            out[fkl_kernel_name(k)] = (n, ms)
    return out


class FusedChunkedKL(torch.autograd.Function):
    """Autograd wrapper. The fused method saves lse and the gathered logits, not
    the N x V logits; with keep=True the forward-chunked variant saves the
    logits instead and its backward skips the recompute."""

    @staticmethod
    def forward(ctx, hidden, weight, topk_idx, topk_logit, T, chunk, keep, row_weight, labels,
                alpha):
        shape = hidden.shape
        h2 = hidden.reshape(-1, shape[-1]).contiguous()
        N = h2.shape[0]
        idx = topk_idx.reshape(N, -1).to(torch.int32).contiguous()
        lg = topk_logit.reshape(N, -1).to(torch.float32).contiguous()
        w = weight.contiguous()
        rw = None if row_weight is None else row_weight.reshape(N).to(torch.float32).contiguous()
        y = None if labels is None else labels.reshape(N).to(torch.int32).contiguous()
        z = None
        if rw is None and y is None:
            if keep:
                out, z = fkl_forward_keep(h2, w, idx, lg, T, chunk)
            else:
                out = fkl_forward(h2, w, idx, lg, T, chunk)
        else:
            res = fkl_forward_ex(h2, w, idx, lg, T, chunk, row_weight=rw, labels=y, alpha=alpha,
                                 keep_logits=True if keep else None)
            out, z = res if keep else (res, None)
        ctx.save_for_backward(h2, w, idx, lg, out.lse, out.topk_z, z, rw, y, out.lse1)
        ctx.T, ctx.chunk, ctx.shape, ctx.alpha = T, chunk, shape, alpha
        # the kept logits are overwritten with G by the backward (through a raw
        # pointer, which torch's version counter does not see): one backward only
        ctx.logits_consumed = False
        return out.loss

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, grad_loss):
        g = grad_loss.to(torch.float32).reshape(()).contiguous()
        h2, w, idx, lg, lse, zk, z, rw, y, lse1 = ctx.saved_tensors
        if z is not None:
            if ctx.logits_consumed:
                raise RuntimeError(
                    "fused_chunked_kl(keep_logits=...): the kept logits were consumed by the "
                    "first backward pass; a second backward through the same graph needs "
                    "keep_logits=False")
            ctx.logits_consumed = True
        if rw is None and y is None:
            if z is not None:
                gh, gw = fkl_backward_keep(h2, w, idx, lg, lse, ctx.T, z, topk_z=zk, grad_loss=g)
            else:
                gh, gw = fkl_backward(h2, w, idx, lg, lse, ctx.T, ctx.chunk, topk_z=zk,
                                      grad_loss=g)
        else:
            gh, gw = fkl_backward_ex(h2, w, idx, lg, lse, ctx.T, ctx.chunk, topk_z=zk, grad_loss=g,
                                     row_weight=rw, labels=y, alpha=ctx.alpha, lse1=lse1,
                                     logits=z)
        return (gh.reshape(ctx.shape), gw.to(w.dtype), None, None, None, None, None, None, None,
                None)


class RenormTopKKL(torch.autograd.Function):
    """Autograd wrapper of the student-renormalised loss: saves the gathered
    student logits; the backward needs no vocabulary-wide work."""

    @staticmethod
    def forward(ctx, hidden, weight, topk_idx, topk_logit, T, row_weight):
        shape = hidden.shape
        h2 = hidden.reshape(-1, shape[-1]).contiguous()
        N = h2.shape[0]
        idx = topk_idx.reshape(N, -1).to(torch.int32).contiguous()
        lg = topk_logit.reshape(N, -1).to(torch.float32).contiguous()
        w = weight.contiguous()
        rw = None if row_weight is None else row_weight.reshape(N).to(torch.float32).contiguous()
        out = fkl_renorm_forward(h2, w, idx, lg, T, row_weight=rw)
        ctx.save_for_backward(h2, w, idx, lg, out.topk_z, rw)
        ctx.T, ctx.shape = T, shape
        return out.loss

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, grad_loss):
        g = grad_loss.to(torch.float32).reshape(()).contiguous()
        h2, w, idx, lg, zk, rw = ctx.saved_tensors
        gh, gw = fkl_renorm_backward(h2, w, idx, lg, ctx.T, topk_z=zk, grad_loss=g, row_weight=rw)
        return gh.reshape(ctx.shape), gw.to(w.dtype), None, None, None, None


def renorm_topk_kl(hidden: torch.Tensor, weight: torch.Tensor, topk_idx: torch.Tensor,
                   topk_logit: torch.Tensor, T: float = 1.0, *,
                   row_weight: torch.Tensor | None = None) -> torch.Tensor:
    """Sum over tokens of w_r T^2 KL(teacher || student) with both softmaxes
    taken over the K cached entries of each token (entries with a -inf teacher
    logit are padding). Shapes as fused_chunked_kl; no chunk parameter, since
    nothing of size N x V is formed."""
    return RenormTopKKL.apply(hidden, weight, topk_idx, topk_logit, float(T), row_weight)


def choose_keep(N: int, d: int, V: int, K: int, dtype: torch.dtype, budget: int | None,
                device=None) -> bool:
    """Memory-budget rule of keep="auto": keep the logits when the kept logits
    plus the keep-mode backward workspace fit in `budget` bytes (default: half
    of the device memory free now)."""
    zb, wb = fkl_keep_sizes(N, d, V, K, dtype)
    if budget is None:
        free, _ = torch.cuda.mem_get_info(device)
        budget = free // 2
    return zb + wb <= budget


def fused_chunked_kl(hidden: torch.Tensor, weight: torch.Tensor, topk_idx: torch.Tensor,
                     topk_logit: torch.Tensor, T: float = 1.0, chunk: int = 2048, *,
                     keep_logits: bool | str = False, memory_budget: int | None = None,
                     row_weight: torch.Tensor | None = None, labels: torch.Tensor | None = None,
                     alpha: float = 0.5) -> torch.Tensor:
    """Sum over tokens of T^2 KL(teacher top-K softmax || student softmax) at temperature T.

    hidden [..., d] (bf16 or fp32), weight [V, d] (LM head, nn.Linear layout),
    topk_idx / topk_logit [..., K]. Returns a 0-d fp32 tensor; gradients flow to
    hidden and weight.

    keep_logits=False is the fused chunked method (memory linear in the tokens,
    logits recomputed in the backward); True keeps the N x V logits for the
    backward (the forward-chunked variant: no recompute, N * V elements more
    memory); "auto" keeps them when they fit in memory_budget bytes (default:
    half of the free device memory).

    row_weight [...] weights each token's term (0 masks padding; mask /
    mask.sum() gives the mean over valid tokens). labels [...] (hard labels,
    < 0 for none) add the cross-entropy at temperature 1: the loss becomes
    sum_r w_r (alpha T^2 KL_r + (1 - alpha) CE_r).
    """
    keep = keep_logits
    if keep == "auto":
        V, d = weight.shape
        N = hidden.numel() // hidden.shape[-1]
        keep = choose_keep(N, d, V, topk_idx.shape[-1], hidden.dtype, memory_budget,
                           hidden.device)
    elif not isinstance(keep, bool):
        raise ValueError(f"keep_logits must be True, False or 'auto' (got {keep_logits!r})")
    return FusedChunkedKL.apply(hidden, weight, topk_idx, topk_logit, float(T), int(chunk),
                                bool(keep), row_weight, labels, float(alpha))
