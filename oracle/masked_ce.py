"""fp64 CPU oracle for sum-reduced masked cross-entropy and fused linear cross-entropy.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously correct statement of
what the GPU path computes. Only the test-suite, the package smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does. It shares no code with the HIP
library and imports nothing from it.

Sources (titles of the pages this follows):
  [CE]   NeMo Automodel PR #2996, "feat(loss): chunked masked CE, packing-mask preservation,
         scoped MoE AC" — first commit message (sum-reduced masked CE: per-row logsumexp,
         label-logit gather, one scalar; softmax recomputed for the gradient; zero
         ``num_label_tokens`` guard), the fourth commit message (the gradient may be written
         over the logits storage) and the *Proof* section (ignore_index holes and a mask,
         parity against ``F.cross_entropy(reduction="sum")``).
  [FLCE] Liger-Kernel issue #533, "Gradient checkpointing for grad_weight in LFCE" — the
         feature pitch (per-chunk logits from input·weightᵀ, a ``[V, H]`` grad_weight updated
         by a matrix multiply-add of the logits gradient and the input chunk) and
         Liger-Kernel issue #941, "No gain in VRAM usage with
         LigerFusedLinearCrossEntropyLoss" — the call signature (hidden, target, lm_head
         weight, optional bias).

The chunked method reaches exactly (up to rounding order) the plain full-tensor result: the
chunks only re-associate a sum. So every function below is that plain definition, written in
fp64 with no chunking, blocking or fusion beyond row blocks that bound host memory (rows are
independent, so a row block changes nothing).

Readings of points the pages leave open (each is repeated in the design notes):
  * T = ``num_label_tokens`` is caller-supplied; when not given, T = number of rows that carry
    a label. The scale is s = 1/T for T > 0 and s = 0 for T = 0 (the zero guard: loss 0 and
    an all-zero gradient, never NaN).
  * A row carries a label when its label differs from ``ignore_index``, lies in [0, V), and
    (if a mask is given) its mask entry is nonzero. A label outside [0, V) that is not
    ``ignore_index`` is treated as ignored and raises the ``bad_label`` flag.
  * The upstream scalar gradient g_out multiplies every gradient (chain rule).
  * Ignored rows have an exactly-zero gradient.
  * FLCE logits are z = h·Wᵀ + b with h and W bf16 values and b float32, all widened exactly
    to fp64.

Parity status: every public function is pinned by tests that do not call this module's
arithmetic (closed forms, textbook special cases, brute force, finite differences, torch's
own cross-entropy and autograd in fp64 on CPU).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16/int16) to float64.

    A bf16 value is the upper half of an IEEE float32, so shifting the 16 bits into the top of
    a 32-bit word gives the float32 with the same value; float32 → float64 is exact.
    """
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def labelled_rows(labels: np.ndarray, v: int, ignore_index: int = -100,
                  mask: np.ndarray | None = None) -> tuple[np.ndarray, bool]:
    """Rows that carry a label, and whether any label was out of range.

    [CE] *Proof* section: rows can be dropped by ignore_index holes and by a mask.
    """
    labels = np.asarray(labels).astype(np.int64)
    not_ignored = labels != ignore_index
    in_range = (labels >= 0) & (labels < v)
    bad = bool(np.any(not_ignored & ~in_range))
    ok = not_ignored & in_range
    if mask is not None:
        ok &= np.asarray(mask) != 0
    return ok, bad


def scale_from_count(t: int) -> float:
    """s = 1/T, with the zero guard of [CE] (first commit message): T = 0 gives s = 0."""
    return 1.0 / float(t) if t > 0 else 0.0


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """Row-wise ln Σ_v exp(z_v), evaluated with the textbook max shift m = max_v z_v."""
    m = np.max(z, axis=1)
    return m + np.log(np.sum(np.exp(z - m[:, None]), axis=1))


@dataclass
class CEResult:
    loss: float           # s · Σ_{labelled i} (lse_i − z_{i,y_i}), times nothing else
    lse: np.ndarray       # fp64 [N]; computed for every row (ignored rows included)
    row_loss: np.ndarray  # fp64 [N]; lse_i − z_{i,y_i} for labelled rows, 0 elsewhere
    count: int            # T actually used
    scale: float          # s
    bad_label: bool
    grad: np.ndarray | None  # fp64 [N, V] (or [len(rows), V] when rows were requested)


def ce_masked_sum(z: np.ndarray, labels: np.ndarray, ignore_index: int = -100,
                  num_label_tokens: int | None = None, mask: np.ndarray | None = None,
                  grad_output: float = 1.0, want_grad: bool = True) -> CEResult:
    """Sum-reduced masked CE over materialised logits ``z`` (fp64 ``[N, V]``).

    [CE] first commit message: the loss is the sum over labelled rows of the row logsumexp
    minus the label logit, divided by ``num_label_tokens``; its gradient is the row softmax
    minus the one-hot label, times the same factor; rows without a label contribute nothing.
    """
    z = np.asarray(z, dtype=np.float64)
    n, v = z.shape
    labels = np.asarray(labels).astype(np.int64)
    ok, bad = labelled_rows(labels, v, ignore_index, mask)
    t = int(ok.sum()) if num_label_tokens is None else int(num_label_tokens)
    s = scale_from_count(t)
    lse = logsumexp_rows(z) if n > 0 else np.zeros(0)
    rows = np.nonzero(ok)[0]
    row_loss = np.zeros(n)
    row_loss[rows] = lse[rows] - z[rows, labels[rows]]
    loss = s * float(np.sum(row_loss))
    grad = None
    if want_grad:
        grad = np.zeros((n, v))
        p = np.exp(z[rows] - lse[rows, None])
        p[np.arange(rows.size), labels[rows]] -= 1.0
        grad[rows] = grad_output * s * p
    return CEResult(loss, lse, row_loss, t, s, bad, grad)


def ce_masked_sum_bits(bits: np.ndarray, labels: np.ndarray, ignore_index: int = -100,
                       num_label_tokens: int | None = None, grad_output: float = 1.0,
                       grad_rows: np.ndarray | None = None, row_block: int = 256) -> CEResult:
    """Same definition as :func:`ce_masked_sum`, read from bf16 bits one row block at a time.

    For logits too large for fp64 in host memory. ``grad_rows`` selects which rows of the
    gradient to return (``None`` = all rows); the loss always covers every row. Each row's
    result depends only on that row, so the blocking does not change any value.
    """
    n, v = bits.shape
    labels = np.asarray(labels).astype(np.int64)
    ok, bad = labelled_rows(labels, v, ignore_index)
    t = int(ok.sum()) if num_label_tokens is None else int(num_label_tokens)
    s = scale_from_count(t)
    lse = np.zeros(n)
    row_loss = np.zeros(n)
    want = np.arange(n) if grad_rows is None else np.asarray(grad_rows, dtype=np.int64)
    grad = np.zeros((want.size, v))
    where = {int(r): k for k, r in enumerate(want)}
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        zb = bf16_bits_to_f64(bits[r0:r1])
        lse[r0:r1] = logsumexp_rows(zb)
        for i in range(r0, r1):
            if ok[i]:
                row_loss[i] = lse[i] - zb[i - r0, labels[i]]
            k = where.get(i)
            if k is not None and ok[i]:
                g = np.exp(zb[i - r0] - lse[i])
                g[labels[i]] -= 1.0
                grad[k] = grad_output * s * g
    loss = s * float(np.sum(row_loss))
    return CEResult(loss, lse, row_loss, t, s, bad, grad)


@dataclass
class FLCEResult:
    loss: float
    lse: np.ndarray            # fp64 [N]
    row_loss: np.ndarray       # fp64 [N]
    count: int
    scale: float
    bad_label: bool
    grad_hidden: np.ndarray | None   # fp64 [N, H] (or the requested rows)
    grad_weight: np.ndarray | None   # fp64 [V, H] (or the requested vocab rows)
    grad_bias: np.ndarray | None     # fp64 [V] (None when there is no bias)


def flce(hidden: np.ndarray, weight: np.ndarray, labels: np.ndarray,
         bias: np.ndarray | None = None, ignore_index: int = -100,
         num_label_tokens: int | None = None, grad_output: float = 1.0,
         grad_weight_init: np.ndarray | None = None, want_grads: bool = True,
         hidden_rows: np.ndarray | None = None, weight_rows: np.ndarray | None = None,
         row_block: int = 256) -> FLCEResult:
    """Fused linear CE as its plain definition: CE of :func:`ce_masked_sum` on z = h·Wᵀ + b.

    [FLCE] issue #533 feature pitch: the logits of a chunk are the input chunk times the
    weight transposed; grad_weight collects (logits gradient)ᵀ · input. Issue #941: the loss
    takes hidden states, targets, the lm_head weight and an optional bias.

    With G = ∂L/∂z (softmax minus one-hot times g_out·s on labelled rows, 0 elsewhere):
    grad_hidden = G·W, grad_weight = Gᵀ·h (+ ``grad_weight_init`` when accumulating into an
    existing buffer, as for tied embeddings), grad_bias = Σ_rows G.

    ``hidden``/``weight`` are fp64 arrays of bf16 values (or raw uint16 bf16 bits, decoded
    here); ``bias`` is float32 or fp64. ``hidden_rows``/``weight_rows`` restrict which rows of
    grad_hidden/grad_weight are returned (the loss always covers all rows).
    """
    h = bf16_bits_to_f64(hidden) if np.asarray(hidden).dtype == np.uint16 else np.asarray(hidden, np.float64)
    w = bf16_bits_to_f64(weight) if np.asarray(weight).dtype == np.uint16 else np.asarray(weight, np.float64)
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    n, hd = h.shape
    v = w.shape[0]
    labels = np.asarray(labels).astype(np.int64)
    ok, bad = labelled_rows(labels, v, ignore_index)
    t = int(ok.sum()) if num_label_tokens is None else int(num_label_tokens)
    s = scale_from_count(t)
    hrows = np.arange(n) if hidden_rows is None else np.asarray(hidden_rows, np.int64)
    wrows = np.arange(v) if weight_rows is None else np.asarray(weight_rows, np.int64)
    hpos = {int(r): k for k, r in enumerate(hrows)}
    lse = np.zeros(n)
    row_loss = np.zeros(n)
    dh = np.zeros((hrows.size, hd)) if want_grads else None
    dw = None
    if want_grads:
        dw = np.zeros((wrows.size, hd))
        if grad_weight_init is not None:
            dw += np.asarray(grad_weight_init, dtype=np.float64)[wrows]
    db = np.zeros(v) if (want_grads and b is not None) else None
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        z = h[r0:r1] @ w.T
        if b is not None:
            z += b[None, :]
        lse_b = logsumexp_rows(z)
        lse[r0:r1] = lse_b
        okb = ok[r0:r1]
        idx = np.nonzero(okb)[0]
        row_loss[r0 + idx] = lse_b[idx] - z[idx, labels[r0 + idx]]
        if not want_grads:
            continue
        g = np.exp(z - lse_b[:, None])
        g[idx, labels[r0 + idx]] -= 1.0
        g[~okb] = 0.0
        g *= grad_output * s
        sel = [(i - r0, hpos[i]) for i in range(r0, r1) if i in hpos]
        if sel:
            src = np.array([a for a, _ in sel])
            dst = np.array([c for _, c in sel])
            dh[dst] = g[src] @ w
        dw += g[:, wrows].T @ h[r0:r1]
        if db is not None:
            db += g.sum(axis=0)
    loss = s * float(np.sum(row_loss))
    return FLCEResult(loss, lse, row_loss, t, s, bad, dh, dw, db)
