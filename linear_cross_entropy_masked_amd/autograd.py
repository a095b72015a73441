"""PyTorch autograd functions over the library's C-ABI calls.

Argument marshalling only: every step of the loss and its gradients runs in the library's
kernels; this module picks the calls, folds a label mask into ignore_index, flattens leading
dimensions, and keeps what the backward needs.

Behaviour follows NeMo Automodel PR #2996 (the masked CE loss with a chunk_size):
  * the forward keeps only the original-dtype logits, the labels and the fp32 lse [n] for
    the backward, which rebuilds the softmax from them (commit messages 1 and 4);
  * writing the gradient into the logits storage is opt-in and keyword-only
    (``inplace_grad=True``; default False, the logits are left intact), the backward is
    once-differentiable, so a double backward raises, and after an in-place backward the
    logits' version counter is bumped, so any other autograd user of the logits fails loudly
    instead of reading the gradient as logits; a second backward through the same graph
    (``retain_graph=True``) raises too, since the logits are gone (seventh commit message:
    the keyword-only opt-in, the once-differentiable backward and the retain_graph hazard);
  * ``reduction``: "sum" is the method's sum over labelled rows, divided by
    ``num_label_tokens`` when it is given; "mean" divides by the number of labelled rows
    (counted on the device); "none" returns the per-row terms (0 for rows without a label).

The fused linear CE function uses the split calls (``flce_fwd`` in the forward, ``flce_bwd``
in the backward): nothing of size [V, H] lives from the forward to the backward (Liger-Kernel
issue #533, feature pitch), and the upstream gradient stays on the device.
"""
from __future__ import annotations

import torch
from torch.autograd.function import once_differentiable

from . import (ce_chunked_bwd, ce_chunked_bwd_inplace, ce_chunked_fwd, ce_rows_bwd, ce_rows_fwd,
               flce_bwd, flce_fwd)

REDUCTIONS = ("sum", "mean", "none")


def _check_reduction(reduction, num_label_tokens, allowed=REDUCTIONS):
    if reduction not in allowed:
        raise ValueError(f"reduction must be one of {allowed}, got {reduction!r}")
    if num_label_tokens is not None and reduction != "sum":
        raise ValueError("num_label_tokens divides the summed loss: use it with reduction='sum'")


def _normaliser(reduction, num_label_tokens):
    """The library's T: the sum is divided by T; -1 asks for the device count of labelled rows."""
    if reduction == "mean":
        return -1
    return 1 if num_label_tokens is None else int(num_label_tokens)


def _flat_labels(labels, mask, n, ignore_index):
    if labels.numel() != n:
        raise ValueError(f"labels has {labels.numel()} entries, expected {n}")
    labels = labels.reshape(n)
    if mask is not None:
        if mask.numel() != n:
            raise ValueError(f"mask has {mask.numel()} entries, expected {n}")
        mask = mask.reshape(n)
        labels = torch.where(mask.to(torch.bool), labels,
                             torch.full_like(labels, ignore_index))
    return labels


class _MaskedCE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, labels, ignore_index, chunk_size, count, reduction, inplace_grad):
        if reduction == "none":
            out, lse = ce_rows_fwd(logits, labels, ignore_index=ignore_index,
                                   chunk_size=chunk_size)
        else:
            out, lse = ce_chunked_fwd(logits, labels, ignore_index=ignore_index,
                                      chunk_size=chunk_size, num_label_tokens=count)
        ctx.save_for_backward(logits, labels, lse)
        ctx.cfg = (ignore_index, chunk_size, count, reduction, inplace_grad)
        ctx.spent = False
        return out

    @staticmethod
    @once_differentiable
    def backward(ctx, g):
        ignore_index, chunk_size, count, reduction, inplace = ctx.cfg
        if inplace and ctx.spent:
            raise RuntimeError(
                "masked CE with inplace_grad=True: the logits were overwritten by the first "
                "backward; a second backward through this graph (retain_graph=True) cannot run")
        logits, labels, lse = ctx.saved_tensors
        if g.dtype != torch.float32:
            g = g.to(torch.float32)
        if reduction == "none":
            grad = ce_rows_bwd(logits, labels, g.contiguous(), inplace=inplace,
                               ignore_index=ignore_index, chunk_size=chunk_size, lse=lse)
        elif inplace:
            grad = ce_chunked_bwd_inplace(logits, labels, ignore_index=ignore_index,
                                          chunk_size=chunk_size, num_label_tokens=count,
                                          grad_output=g, lse=lse)
        else:
            grad = ce_chunked_bwd(logits, labels, ignore_index=ignore_index,
                                  chunk_size=chunk_size, num_label_tokens=count,
                                  grad_output=g, lse=lse)
        if inplace:
            ctx.spent = True
            torch.autograd.graph.increment_version(logits)
        return grad, None, None, None, None, None, None


def masked_cross_entropy(logits, labels, *, mask=None, ignore_index: int = -100,
                         chunk_size: int = 1024, num_label_tokens: int | None = None,
                         reduction: str = "sum", inplace_grad: bool = False):
    """Masked CE over bf16 logits [..., V] with int labels [...]: a 0-d fp32 loss ("sum",
    "mean") or fp32 per-row terms of the leading shape ("none"). ``mask`` (same leading
    shape, nonzero = keep) is folded into the labels as ignore_index."""
    _check_reduction(reduction, num_label_tokens)
    if logits.dim() < 1:
        raise ValueError("logits must have a vocabulary dimension")
    lead = logits.shape[:-1]
    v = logits.shape[-1]
    flat = logits.view(-1, v)  # a view (never a copy), so an in-place gradient lands in logits
    n = flat.shape[0]
    lab = _flat_labels(labels, mask, n, ignore_index)
    out = _MaskedCE.apply(flat, lab, int(ignore_index), int(chunk_size),
                          _normaliser(reduction, num_label_tokens), reduction, bool(inplace_grad))
    return out.view(lead) if reduction == "none" else out


class MaskedCrossEntropy(torch.nn.Module):
    """Module form of :func:`masked_cross_entropy` (the constructor arguments of the masked CE
    loss in NeMo Automodel PR #2996: chunk_size, and inplace_grad keyword-only, default
    False)."""

    def __init__(self, *, ignore_index: int = -100, chunk_size: int = 1024,
                 reduction: str = "sum", inplace_grad: bool = False):
        super().__init__()
        _check_reduction(reduction, None)
        self.ignore_index = ignore_index
        self.chunk_size = chunk_size
        self.reduction = reduction
        self.inplace_grad = inplace_grad

    def forward(self, logits, labels, mask=None, num_label_tokens=None):
        return masked_cross_entropy(logits, labels, mask=mask, ignore_index=self.ignore_index,
                                    chunk_size=self.chunk_size,
                                    num_label_tokens=num_label_tokens,
                                    reduction=self.reduction, inplace_grad=self.inplace_grad)


class _LinearCE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, bias, labels, ignore_index, chunk_size, count, grad_buffer):
        loss, lse = flce_fwd(hidden, weight, labels, bias, ignore_index=ignore_index,
                             chunk_size=chunk_size, num_label_tokens=count)
        ctx.save_for_backward(hidden, weight, bias, labels, lse)
        ctx.cfg = (ignore_index, chunk_size, count, grad_buffer)
        return loss

    @staticmethod
    @once_differentiable
    def backward(ctx, g):
        ignore_index, chunk_size, count, grad_buffer = ctx.cfg
        hidden, weight, bias, labels, lse = ctx.saved_tensors
        if g.dtype != torch.float32:
            g = g.to(torch.float32)
        need_h, need_w, need_b = ctx.needs_input_grad[:3]
        need_b = bool(need_b and bias is not None)
        to_buffer = grad_buffer is not None and need_w
        # each output: True = allocate, False = not computed, a tensor = written (or, with
        # accumulate, added) in place. The accumulate flag covers grad_bias too, so with the
        # weight buffer the bias gradient is added into a zeroed tensor of its own.
        gb_spec = need_b
        if to_buffer and need_b:
            gb_spec = torch.zeros(bias.shape[0], dtype=torch.float32, device=bias.device)
        gh, gw, gb = flce_bwd(
            hidden, weight, labels, lse, bias, ignore_index=ignore_index, chunk_size=chunk_size,
            num_label_tokens=count, grad_output=g, accumulate=to_buffer,
            grad_hidden=bool(need_h), grad_weight=grad_buffer if to_buffer else bool(need_w),
            grad_bias=gb_spec)
        return (gh if need_h else None,
                None if (to_buffer or not need_w) else gw,
                gb if need_b else None,
                None, None, None, None, None)


def linear_cross_entropy(hidden, weight, labels, bias=None, *, mask=None,
                         ignore_index: int = -100, chunk_size: int = 1024,
                         num_label_tokens: int | None = None, reduction: str = "sum",
                         weight_grad_buffer=None):
    """Fused linear CE: loss of logits = hidden · weightᵀ (+ bias) without materialising them.
    hidden bf16 [..., H], weight bf16 [V, H], bias fp32 [V] or None, labels [...].

    The weight gradient is computed into an fp32 accumulator; autograd hands it to ``weight``
    in the weight's dtype. With ``weight_grad_buffer`` (fp32 [V, H]) it is instead added into
    that buffer and ``weight.grad`` is left alone (an fp32 main-gradient, or tied embeddings).
    reduction: "sum" or "mean" (per-row terms are not offered for the fused layer)."""
    _check_reduction(reduction, num_label_tokens, allowed=("sum", "mean"))
    if weight_grad_buffer is not None:
        if (weight_grad_buffer.dtype != torch.float32
                or tuple(weight_grad_buffer.shape) != tuple(weight.shape)
                or not weight_grad_buffer.is_contiguous()):
            raise ValueError("weight_grad_buffer must be a contiguous fp32 tensor of the "
                             "weight's shape")
    h = hidden.shape[-1]
    flat = hidden.reshape(-1, h)
    n = flat.shape[0]
    lab = _flat_labels(labels, mask, n, ignore_index)
    return _LinearCE.apply(flat, weight, bias, lab, int(ignore_index), int(chunk_size),
                           _normaliser(reduction, num_label_tokens), weight_grad_buffer)


class LinearCrossEntropy(torch.nn.Module):
    """Module form of :func:`linear_cross_entropy` (the weight and bias are passed in, as with
    a tied lm_head)."""

    def __init__(self, *, ignore_index: int = -100, chunk_size: int = 1024,
                 reduction: str = "sum"):
        super().__init__()
        _check_reduction(reduction, None, allowed=("sum", "mean"))
        self.ignore_index = ignore_index
        self.chunk_size = chunk_size
        self.reduction = reduction

    def forward(self, hidden, weight, labels, bias=None, mask=None, num_label_tokens=None,
                weight_grad_buffer=None):
        return linear_cross_entropy(hidden, weight, labels, bias, mask=mask,
                                    ignore_index=self.ignore_index, chunk_size=self.chunk_size,
                                    num_label_tokens=num_label_tokens, reduction=self.reduction,
                                    weight_grad_buffer=weight_grad_buffer)


def ce_chunked(logits, labels, *, mask=None, ignore_index: int = -100, chunk_size: int = 1024,
               num_label_tokens: int | None = None, inplace_grad: bool = False):
    """The masked CE loss under the name and defaults of the library's interface: the sum over
    labelled rows divided by T = num_label_tokens, or by the number of labelled rows (counted
    on the device) when it is None; gradient out of place unless inplace_grad=True."""
    if num_label_tokens is None:
        return masked_cross_entropy(logits, labels, mask=mask, ignore_index=ignore_index,
                                    chunk_size=chunk_size, reduction="mean",
                                    inplace_grad=inplace_grad)
    return masked_cross_entropy(logits, labels, mask=mask, ignore_index=ignore_index,
                                chunk_size=chunk_size, num_label_tokens=num_label_tokens,
                                reduction="sum", inplace_grad=inplace_grad)


def flce(hidden, weight, labels, bias=None, *, mask=None, ignore_index: int = -100,
         chunk_size: int = 1024, num_label_tokens: int | None = None, recompute: bool = True,
         weight_grad_buffer=None):
    """The fused linear CE loss under the name and defaults of the library's interface (T as in
    :func:`ce_chunked`). Under autograd the backward always rebuilds the logits from the saved
    lse (nothing of size [N, V] or [V, H] lives between forward and backward), i.e. the
    recomputing schedule; ``recompute=False`` (keep the fp32 slice, one logits product fewer)
    is the fused call ``flce_fwd_bwd`` when the upstream gradient is known, not an autograd
    schedule, and is refused here."""
    if not recompute:
        raise ValueError("flce under autograd always recomputes; call flce_fwd_bwd for the "
                         "stored-slice schedule")
    reduction = "mean" if num_label_tokens is None else "sum"
    return linear_cross_entropy(hidden, weight, labels, bias, mask=mask,
                                ignore_index=ignore_index, chunk_size=chunk_size,
                                num_label_tokens=num_label_tokens, reduction=reduction,
                                weight_grad_buffer=weight_grad_buffer)
