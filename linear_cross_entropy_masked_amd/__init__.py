"""Thin Python binding of liblce_masked.so (the C-ABI in include/lce_masked.h).

Argument marshalling only: this module checks dtypes/devices, allocates outputs and the
workspace through PyTorch (device memory and streams are all PyTorch provides here), and
calls the C entry points of the same names on the current HIP stream. Every step of the loss
runs in the library's HIP kernels; there is no CPU or PyTorch fallback, and importing a
function whose library is missing raises.

Entry points (same names as the C ABI):
    ce_chunked_fwd, ce_chunked_bwd, ce_chunked_bwd_inplace, flce_fwd_bwd, flce_fwd, flce_bwd,
    ce_chunked_workspace_size, flce_workspace_size, lce_status_str
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LceError", "library_path", "load_library",
    "ce_chunked_workspace_size", "ce_chunked_fwd", "ce_chunked_bwd", "ce_chunked_bwd_inplace",
    "ce_chunked_fwd_bwd_inplace", "ce_chunked_fwd_bwd_inplace_noalloc", "ce_rows_fwd",
    "ce_rows_bwd", "LCE_NOALLOC_MAX_ROWS",
    "flce_workspace_size", "flce_fwd_bwd", "flce_fwd", "flce_bwd", "lce_status_str",
    "flce_status_str",
    "FLCE_RECOMPUTE", "FLCE_ACCUMULATE", "LCE_STATUS_BAD_LABEL",
    "lce_timing_enable", "lce_timing_read",
]

FLCE_RECOMPUTE = 1
FLCE_ACCUMULATE = 2
LCE_STATUS_BAD_LABEL = 1
LCE_NOALLOC_MAX_ROWS = 1 << 20  # rows the allocation-free CE step's static scratch holds

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class LceError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed with status {code}: {lce_status_str(code)}")
        self.code = code


def library_path() -> str:
    return os.environ.get("LCE_MASKED_LIB", os.path.join(_PKG, "liblce_masked.so"))


def load_library() -> ctypes.CDLL:
    """Load (once) and return the C-ABI library; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m linear_cross_entropy_masked_amd.build` "
            "(the HIP library is the only implementation; there is no fallback)")
    lib = ctypes.CDLL(path)
    i64, i32, u32, sz, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p
    psz = ctypes.POINTER(ctypes.c_size_t)
    sigs = {
        "lce_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "flce_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "ce_chunked_workspace_size": (ctypes.c_int, [i64, i64, i64, psz]),
        "ce_chunked_fwd": (ctypes.c_int, [vp, i64, i64, i64, vp, i32, i64, i64, vp, vp, vp, vp, sz, vp]),
        "ce_chunked_bwd": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, vp, i32, i64, i64, vp, vp, vp, vp, sz, vp]),
        "ce_chunked_bwd_inplace": (ctypes.c_int, [vp, i64, i64, i64, vp, i32, i64, i64, vp, vp, vp, vp, sz, vp]),
        "ce_chunked_fwd_bwd_inplace": (ctypes.c_int, [vp, i64, i64, i64, vp, i32, i64, i64, vp, vp, vp,
                                                      vp, vp, sz, vp]),
        "ce_chunked_fwd_bwd_inplace_noalloc": (ctypes.c_int, [vp, i64, i64, i64, vp, i32, i64, i64,
                                                              vp, vp, vp, vp, vp]),
        "ce_rows_fwd": (ctypes.c_int, [vp, i64, i64, i64, vp, i32, i64, vp, vp, vp, vp, sz, vp]),
        "ce_rows_bwd": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, vp, i32, i64, vp, vp, vp, vp, sz,
                                       vp]),
        "flce_workspace_size": (ctypes.c_int, [i64, i64, i64, i64, u32, psz]),
        "flce_fwd_bwd": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, i64, i32, i64, i64, u32, vp, vp, vp,
                                        vp, vp, vp, vp, vp, sz, vp]),
        "flce_fwd": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, i64, i32, i64, i64, vp, vp, vp, vp,
                                    sz, vp]),
        "flce_bwd": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, i64, u32, vp, vp,
                                    vp, vp, vp, vp, sz, vp]),
        "lce_timing_enable": (ctypes.c_int, [ctypes.c_int]),
        "lce_timing_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                           ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_longlong),
                                           ctypes.POINTER(ctypes.c_int)]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIB = lib
    return lib


def lce_status_str(code: int) -> str:
    return load_library().lce_status_str(int(code)).decode()


def flce_status_str(code: int) -> str:
    return load_library().flce_status_str(int(code)).decode()


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise LceError(fn, code)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, name, dtype, dims, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimension(s), got shape {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _labels_i32(labels, n, device, ignore_index=-100):
    """int32 labels for the C ABI. An int64 label outside the int32 range is not a vocabulary
    index: it becomes a negative value other than ignore_index, so the library flags it
    (LCE_STATUS_BAD_LABEL) and treats the row as unlabelled instead of wrapping it onto a
    class."""
    import torch
    _require(labels, "labels", None, 1, device)
    if labels.shape[0] != n:
        raise ValueError(f"labels has {labels.shape[0]} entries, expected {n}")
    if labels.dtype == torch.int64:
        bad = -1 if int(ignore_index) != -1 else -2
        wide = (labels > 2 ** 31 - 1) | (labels < -(2 ** 31))
        labels = torch.where(wide, torch.full_like(labels, bad), labels).to(torch.int32)
    elif labels.dtype != torch.int32:
        raise TypeError("labels must be int32 or int64")
    return labels.contiguous()


def _require_lse(lse, n, device):
    import torch
    _require(lse, "lse", torch.float32, 1, device)
    if lse.shape[0] != n or (n > 1 and lse.stride(0) != 1):
        raise ValueError(f"lse must be a contiguous float32 [{n}] tensor, got shape "
                         f"{tuple(lse.shape)} stride {tuple(lse.stride())}")


def _workspace(nbytes, device, workspace=None):
    import torch
    if workspace is not None:
        if workspace.device != device or workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace must hold at least {nbytes} bytes on {device}")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _count_arg(num_label_tokens):
    return -1 if num_label_tokens is None else int(num_label_tokens)


def ce_chunked_workspace_size(n: int, v: int, chunk_size: int) -> int:
    out = ctypes.c_size_t()
    _check("ce_chunked_workspace_size",
           load_library().ce_chunked_workspace_size(n, v, chunk_size, ctypes.byref(out)))
    return out.value


def flce_workspace_size(n: int, h: int, v: int, chunk_size: int, flags: int = 0) -> int:
    out = ctypes.c_size_t()
    _check("flce_workspace_size",
           load_library().flce_workspace_size(n, h, v, chunk_size, flags, ctypes.byref(out)))
    return out.value


def _logits_2d(logits):
    import torch
    _require(logits, "logits", torch.bfloat16, 2)
    n, v = logits.shape
    if n == 0 or v == 0:
        return n, v, v
    if logits.stride(1) != 1 and v > 1:
        raise ValueError("logits rows must be contiguous (stride(1) == 1)")
    return n, v, (logits.stride(0) if n > 1 else v)


def ce_chunked_fwd(logits, labels, *, ignore_index: int = -100, chunk_size: int = 1024,
                   num_label_tokens: int | None = None, return_lse: bool = True,
                   status=None, workspace=None):
    """Sum-reduced masked CE forward. Returns (loss fp32 0-d tensor, lse fp32 [n] or None)."""
    import torch
    lib = load_library()
    n, v, ld = _logits_2d(logits)
    dev = logits.device
    labels = _labels_i32(labels, n, dev, ignore_index)
    nbytes = ce_chunked_workspace_size(n, v, chunk_size)
    ws = _workspace(nbytes, dev, workspace)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev) if return_lse else None
    _check("ce_chunked_fwd", lib.ce_chunked_fwd(
        _ptr(logits), n, v, ld, _ptr(labels), ignore_index, chunk_size,
        _count_arg(num_label_tokens), _ptr(loss), _ptr(lse), _ptr(status), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(dev)))
    return loss, lse


def ce_chunked_bwd(logits, labels, *, out=None, ignore_index: int = -100, chunk_size: int = 1024,
                   num_label_tokens: int | None = None, grad_output=None, lse=None, status=None,
                   workspace=None):
    """Out-of-place backward: returns grad (bf16, shape of logits); logits are left intact."""
    import torch
    lib = load_library()
    n, v, ld = _logits_2d(logits)
    dev = logits.device
    labels = _labels_i32(labels, n, dev, ignore_index)
    if out is None:
        out = torch.empty((n, v), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, 2, dev)
    if tuple(out.shape) != (n, v) or (n > 0 and v > 1 and out.stride(1) != 1):
        raise ValueError("out must be [n, v] bf16 with contiguous rows")
    ldg = out.stride(0) if n > 1 else v
    if grad_output is not None:
        _require(grad_output, "grad_output", torch.float32, 0, dev)
    if lse is not None:
        _require_lse(lse, n, dev)
    ws = _workspace(ce_chunked_workspace_size(n, v, chunk_size), dev, workspace)
    _check("ce_chunked_bwd", lib.ce_chunked_bwd(
        _ptr(logits), n, v, ld, _ptr(out), ldg, _ptr(labels), ignore_index, chunk_size,
        _count_arg(num_label_tokens), _ptr(grad_output), _ptr(lse), _ptr(status), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(dev)))
    return out


def ce_chunked_bwd_inplace(logits, labels, *, ignore_index: int = -100, chunk_size: int = 1024,
                           num_label_tokens: int | None = None, grad_output=None, lse=None,
                           status=None, workspace=None):
    """In-place backward: overwrites ``logits`` with the gradient and returns it."""
    import torch
    lib = load_library()
    n, v, ld = _logits_2d(logits)
    dev = logits.device
    labels = _labels_i32(labels, n, dev, ignore_index)
    if grad_output is not None:
        _require(grad_output, "grad_output", torch.float32, 0, dev)
    if lse is not None:
        _require_lse(lse, n, dev)
    ws = _workspace(ce_chunked_workspace_size(n, v, chunk_size), dev, workspace)
    _check("ce_chunked_bwd_inplace", lib.ce_chunked_bwd_inplace(
        _ptr(logits), n, v, ld, _ptr(labels), ignore_index, chunk_size,
        _count_arg(num_label_tokens), _ptr(grad_output), _ptr(lse), _ptr(status), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(dev)))
    return logits


def ce_chunked_fwd_bwd_inplace(logits, labels, *, ignore_index: int = -100,
                               chunk_size: int = 1024, num_label_tokens: int | None = None,
                               grad_output=None, return_lse: bool = False, status=None,
                               workspace=None):
    """Forward and in-place backward in one call (the upstream gradient is known now).

    Overwrites ``logits`` with the gradient; returns (loss fp32 0-d tensor, lse fp32 [n] or
    None). Bitwise equal to ``ce_chunked_fwd`` followed by ``ce_chunked_bwd_inplace``."""
    import torch
    lib = load_library()
    n, v, ld = _logits_2d(logits)
    dev = logits.device
    labels = _labels_i32(labels, n, dev, ignore_index)
    if grad_output is not None:
        _require(grad_output, "grad_output", torch.float32, 0, dev)
    ws = _workspace(ce_chunked_workspace_size(n, v, chunk_size), dev, workspace)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev) if return_lse else None
    _check("ce_chunked_fwd_bwd_inplace", lib.ce_chunked_fwd_bwd_inplace(
        _ptr(logits), n, v, ld, _ptr(labels), ignore_index, chunk_size,
        _count_arg(num_label_tokens), _ptr(grad_output), _ptr(loss), _ptr(lse), _ptr(status),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return loss, lse


def ce_chunked_fwd_bwd_inplace_noalloc(logits, labels, *, ignore_index: int = -100,
                                       chunk_size: int = 1024,
                                       num_label_tokens: int | None = None, grad_output=None,
                                       loss=None, lse=None, status=None):
    """:func:`ce_chunked_fwd_bwd_inplace` without a workspace: the library keeps the step's
    O(n) scratch in a static per-GPU array (n <= LCE_NOALLOC_MAX_ROWS). Pass ``loss`` (fp32
    0-d) and optionally ``lse`` (fp32 [n]) to have nothing allocated here either; calls that
    may overlap on one GPU must be serialised by the caller. Returns (loss, lse)."""
    import torch
    lib = load_library()
    n, v, ld = _logits_2d(logits)
    dev = logits.device
    labels = _labels_i32(labels, n, dev, ignore_index)
    if grad_output is not None:
        _require(grad_output, "grad_output", torch.float32, 0, dev)
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    _require(loss, "loss", torch.float32, 0, dev)
    if lse is not None:
        _require_lse(lse, n, dev)
    _check("ce_chunked_fwd_bwd_inplace_noalloc", lib.ce_chunked_fwd_bwd_inplace_noalloc(
        _ptr(logits), n, v, ld, _ptr(labels), ignore_index, chunk_size,
        _count_arg(num_label_tokens), _ptr(grad_output), _ptr(loss), _ptr(lse), _ptr(status),
        _stream(dev)))
    return loss, lse


def ce_rows_fwd(logits, labels, *, ignore_index: int = -100, chunk_size: int = 1024,
                return_lse: bool = True, status=None, workspace=None):
    """Unreduced forward. Returns (row_loss fp32 [n], lse fp32 [n] or None); rows without a
    label get 0."""
    import torch
    lib = load_library()
    n, v, ld = _logits_2d(logits)
    dev = logits.device
    labels = _labels_i32(labels, n, dev, ignore_index)
    ws = _workspace(ce_chunked_workspace_size(n, v, chunk_size), dev, workspace)
    rows = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev) if return_lse else None
    _check("ce_rows_fwd", lib.ce_rows_fwd(
        _ptr(logits), n, v, ld, _ptr(labels), ignore_index, chunk_size, _ptr(rows), _ptr(lse),
        _ptr(status), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return rows, lse


def ce_rows_bwd(logits, labels, grad_rows, *, out=None, inplace: bool = False,
                ignore_index: int = -100, chunk_size: int = 1024, lse=None, status=None,
                workspace=None):
    """Unreduced backward: row i of the result is grad_rows[i] · (softmax − onehot). With
    ``inplace`` the gradient overwrites ``logits``; otherwise it goes to ``out`` (or a new
    tensor)."""
    import torch
    lib = load_library()
    n, v, ld = _logits_2d(logits)
    dev = logits.device
    labels = _labels_i32(labels, n, dev, ignore_index)
    _require(grad_rows, "grad_rows", torch.float32, 1, dev)
    if grad_rows.numel() != n or (n > 1 and grad_rows.stride(0) != 1):
        raise ValueError("grad_rows must be a contiguous fp32 [n] tensor")
    if lse is not None:
        _require_lse(lse, n, dev)
    if inplace:
        out, ldg = logits, ld
    else:
        if out is None:
            out = torch.empty((n, v), dtype=torch.bfloat16, device=dev)
        _require(out, "out", torch.bfloat16, 2, dev)
        if tuple(out.shape) != (n, v) or (n > 0 and v > 1 and out.stride(1) != 1):
            raise ValueError("out must be [n, v] bf16 with contiguous rows")
        ldg = out.stride(0) if n > 1 else v
    ws = _workspace(ce_chunked_workspace_size(n, v, chunk_size), dev, workspace)
    _check("ce_rows_bwd", lib.ce_rows_bwd(
        _ptr(logits), n, v, ld, _ptr(out), ldg, _ptr(labels), ignore_index, chunk_size,
        _ptr(grad_rows), _ptr(lse), _ptr(status), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(dev)))
    return out


def flce_fwd_bwd(hidden, weight, labels, bias=None, *, ignore_index: int = -100,
                 chunk_size: int = 1024, num_label_tokens: int | None = None,
                 recompute: bool = False, accumulate: bool = False, grad_output=None,
                 grad_hidden=True, grad_weight=True, grad_bias=None, return_lse=False,
                 status=None, workspace=None):
    """Fused linear CE forward+backward.

    ``grad_hidden`` / ``grad_weight`` / ``grad_bias``: True to allocate, False/None to skip, or
    a tensor to write into (required for ``accumulate``). grad_bias defaults to True when a
    bias is given. Returns (loss, grad_hidden, grad_weight, grad_bias, lse).
    """
    import torch
    lib = load_library()
    _require(hidden, "hidden", torch.bfloat16, 2)
    dev = hidden.device
    _require(weight, "weight", torch.bfloat16, 2, dev)
    n, h = hidden.shape
    v, h2 = weight.shape
    if h2 != h:
        raise ValueError(f"hidden has {h} columns but weight has {h2}")
    hidden = hidden.contiguous()
    weight = weight.contiguous()
    labels = _labels_i32(labels, n, dev, ignore_index)
    if bias is not None:
        _require(bias, "bias", torch.float32, 1, dev)
        if bias.shape[0] != v:
            raise ValueError("bias must have v entries")
        bias = bias.contiguous()
    if grad_bias is None:
        grad_bias = bias is not None
    flags = (FLCE_RECOMPUTE if recompute else 0) | (FLCE_ACCUMULATE if accumulate else 0)

    def out(spec, shape, dtype, name):
        if spec is True:
            if accumulate and name != "grad_hidden":
                raise ValueError(f"accumulate=True needs an existing {name} tensor")
            return torch.empty(shape, dtype=dtype, device=dev)
        if spec is False or spec is None:
            return None
        _require(spec, name, dtype, len(shape), dev)
        if tuple(spec.shape) != tuple(shape) or not spec.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {tuple(shape)} {dtype} tensor")
        return spec

    gh = out(grad_hidden, (n, h), torch.bfloat16, "grad_hidden")
    gw = out(grad_weight, (v, h), torch.float32, "grad_weight")
    gb = out(grad_bias, (v,), torch.float32, "grad_bias")
    if grad_output is not None:
        _require(grad_output, "grad_output", torch.float32, 0, dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev) if return_lse else None
    ws = _workspace(flce_workspace_size(n, h, v, chunk_size, flags), dev, workspace)
    _check("flce_fwd_bwd", lib.flce_fwd_bwd(
        _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(labels), n, h, v, ignore_index, chunk_size,
        _count_arg(num_label_tokens), flags, _ptr(grad_output), _ptr(loss), _ptr(lse), _ptr(gh),
        _ptr(gw), _ptr(gb), _ptr(status), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(dev)))
    return loss, gh, gw, gb, lse


def _flce_inputs(hidden, weight, labels, bias, ignore_index):
    import torch
    _require(hidden, "hidden", torch.bfloat16, 2)
    dev = hidden.device
    _require(weight, "weight", torch.bfloat16, 2, dev)
    n, h = hidden.shape
    v, h2 = weight.shape
    if h2 != h:
        raise ValueError(f"hidden has {h} columns but weight has {h2}")
    labels = _labels_i32(labels, n, dev, ignore_index)
    if bias is not None:
        _require(bias, "bias", torch.float32, 1, dev)
        if bias.shape[0] != v:
            raise ValueError("bias must have v entries")
        bias = bias.contiguous()
    return hidden.contiguous(), weight.contiguous(), labels, bias, dev, n, h, v


def flce_fwd(hidden, weight, labels, bias=None, *, ignore_index: int = -100,
             chunk_size: int = 1024, num_label_tokens: int | None = None, status=None,
             workspace=None):
    """Fused linear CE forward only. Returns (loss, lse); keep lse for :func:`flce_bwd`."""
    import torch
    lib = load_library()
    hidden, weight, labels, bias, dev, n, h, v = _flce_inputs(
        hidden, weight, labels, bias, ignore_index)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    ws = _workspace(flce_workspace_size(n, h, v, chunk_size, 0), dev, workspace)
    _check("flce_fwd", lib.flce_fwd(
        _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(labels), n, h, v, ignore_index, chunk_size,
        _count_arg(num_label_tokens), _ptr(loss), _ptr(lse), _ptr(status), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(dev)))
    return loss, lse


def flce_bwd(hidden, weight, labels, lse, bias=None, *, ignore_index: int = -100,
             chunk_size: int = 1024, num_label_tokens: int | None = None,
             accumulate: bool = False, grad_output=None, grad_hidden=True, grad_weight=True,
             grad_bias=None, status=None, workspace=None):
    """Fused linear CE backward from :func:`flce_fwd`'s lse (the logits are recomputed).
    Output arguments as in :func:`flce_fwd_bwd`. Returns (grad_hidden, grad_weight, grad_bias)."""
    import torch
    lib = load_library()
    hidden, weight, labels, bias, dev, n, h, v = _flce_inputs(
        hidden, weight, labels, bias, ignore_index)
    _require(lse, "lse", torch.float32, 1, dev)
    if lse.shape[0] != n or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous [n] float32 tensor")
    if grad_bias is None:
        grad_bias = bias is not None
    flags = FLCE_ACCUMULATE if accumulate else 0

    def out(spec, shape, dtype, name):
        if spec is True:
            if accumulate and name != "grad_hidden":
                raise ValueError(f"accumulate=True needs an existing {name} tensor")
            return torch.empty(shape, dtype=dtype, device=dev)
        if spec is False or spec is None:
            return None
        _require(spec, name, dtype, len(shape), dev)
        if tuple(spec.shape) != tuple(shape) or not spec.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {tuple(shape)} {dtype} tensor")
        return spec

    gh = out(grad_hidden, (n, h), torch.bfloat16, "grad_hidden")
    gw = out(grad_weight, (v, h), torch.float32, "grad_weight")
    gb = out(grad_bias, (v,), torch.float32, "grad_bias")
    if grad_output is not None:
        _require(grad_output, "grad_output", torch.float32, 0, dev)
    ws = _workspace(flce_workspace_size(n, h, v, chunk_size, flags), dev, workspace)
    _check("flce_bwd", lib.flce_bwd(
        _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(labels), _ptr(lse), n, h, v, ignore_index,
        chunk_size, _count_arg(num_label_tokens), flags, _ptr(grad_output), _ptr(gh), _ptr(gw),
        _ptr(gb), _ptr(status), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return gh, gw, gb


def lce_timing_enable(on: bool = True) -> None:
    """Bracket every library launch with hipEvents (measurement aid; off by default)."""
    _check("lce_timing_enable", load_library().lce_timing_enable(1 if on else 0))


def lce_timing_read() -> list[tuple[str, float, int]]:
    """(kernel name, total ms, launches) per kernel since the previous read; resets totals."""
    lib = load_library()
    cap = 32
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    cnt = (ctypes.c_longlong * cap)()
    k = ctypes.c_int()
    _check("lce_timing_read", lib.lce_timing_read(cap, names, ms, cnt, ctypes.byref(k)))
    return [(names[i].decode(), ms[i], cnt[i]) for i in range(min(k.value, cap))]
