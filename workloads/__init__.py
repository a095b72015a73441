"""Seeded synthetic inputs for the masked cross-entropy hot path.

This module only draws random inputs and rounds them to bf16 bit patterns. It holds
none of the loss arithmetic: the oracle and the HIP path both consume what it returns
(raw bf16 bits as ``uint16``, labels as ``int32``, bias as ``float32``) and each decodes
the bits on its own side.

Workloads follow the shapes the pages discuss:
  * the chunked masked CE of NeMo Automodel PR #2996 ("feat(loss): chunked masked CE,
    packing-mask preservation, scoped MoE AC"), whose fourth commit message measures
    ``[16384, 128256]`` bf16 logits;
  * the fused linear CE of Liger-Kernel issues #533 ("Gradient checkpointing for grad_weight
    in LFCE") and #941 ("No gain in VRAM usage with LigerFusedLinearCrossEntropyLoss"),
    the latter reporting a V=32777, hidden 768 model;
  * a Llama3-8B-shaped head (hidden 4096, V=128256) as in torchtitan PR #996 ("chunked cross
    entropy loss to reduce peak memory").

Recipe (fixed, so both sides see identical bits):
  * Dense tensors are drawn in blocks of ``BLOCK_ROWS`` rows; block ``b`` of tensor ``t`` uses
    ``PCG64(SeedSequence([seed, wid, t, b]))`` and ``standard_normal(float32) * sigma`` (a
    float32 multiply), then round-to-nearest-even to bf16.
  * Labels, spike rows, ignored rows and document cuts come from one stream
    ``PCG64(SeedSequence([seed, wid, 99]))``, drawn in exactly that order.
  * The ignored count is ``round(frac * N)`` (exact, rows drawn without replacement).
  * A logit spike is added in float32 before the bf16 rounding.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_ROWS = 512
IGNORE_INDEX = -100

# tensor ids used in the seed sequences
_T_LOGITS, _T_HIDDEN, _T_WEIGHT, _T_BIAS = 0, 1, 2, 3
_LABEL_STREAM = 99


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # workload id folded into every seed sequence
    kind: str           # "ce" (materialised logits) or "flce" (hidden @ weight^T)
    n: int
    v: int
    chunk_size: int
    h: int = 0
    logit_sigma: float = 0.0
    spike: float = 0.0
    spike_frac: float = 0.0
    ignore_frac: float = 0.0
    hidden_sigma: float = 1.0
    weight_sigma: float = 0.0
    bias_sigma: float = 0.0     # 0 => no bias
    documents: int = 0          # >0 => packed documents; first label of each is ignored
    recompute: bool = False
    notes: str = field(default="", compare=False)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("ce_64x1000", 1, "ce", n=64, v=1000, chunk_size=16, logit_sigma=2.0,
                 ignore_frac=0.10,
                 notes="small chunked masked CE, fwd+bwd in place"),
        Workload("ce_16384x128256", 2, "ce", n=16384, v=128256, chunk_size=1024,
                 logit_sigma=3.0, spike=8.0, spike_frac=0.30, ignore_frac=0.05,
                 notes="large-vocab chunked masked CE, fwd+bwd in place"),
        Workload("flce_2048x768x32777", 3, "flce", n=2048, h=768, v=32777, chunk_size=512,
                 hidden_sigma=1.0, weight_sigma=0.02, bias_sigma=0.01, ignore_frac=0.02,
                 notes="small-model fused linear CE with bias, V not a multiple of 16"),
        Workload("flce_8192x4096x128256", 4, "flce", n=8192, h=4096, v=128256,
                 chunk_size=1024, hidden_sigma=1.0, weight_sigma=0.02, ignore_frac=0.05,
                 notes="Llama3-8B-shaped head fused linear CE, no bias"),
        Workload("flce_32768x8192x128256_packed", 5, "flce", n=32768, h=8192, v=128256,
                 chunk_size=2048, hidden_sigma=1.0, weight_sigma=0.015, documents=8,
                 recompute=True,
                 notes="long-context packed fused linear CE, full recompute"),
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite normal draws; NaN handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(seed: int, wid: int, tensor: int, rows: int, cols: int, sigma: float,
                spikes: tuple[np.ndarray, np.ndarray, float] | None = None) -> np.ndarray:
    """Blocked N(0, sigma^2) draw rounded to bf16, returned as uint16 ``[rows, cols]``.

    ``spikes`` = (row indices, column indices, value) adds ``value`` in float32 at those
    positions before rounding.
    """
    out = np.empty((rows, cols), dtype=np.uint16)
    nblocks = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    if spikes is not None:
        srows, scols, sval = spikes
        order = np.argsort(srows, kind="stable")
        srows, scols = srows[order], scols[order]

    def fill(b: int) -> None:
        r0 = b * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, tensor, b])))
        x = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        x *= np.float32(sigma)
        if spikes is not None:
            lo, hi = np.searchsorted(srows, [r0, r1])
            if hi > lo:
                x[srows[lo:hi] - r0, scols[lo:hi]] += np.float32(sval)
        out[r0:r1] = f32_to_bf16_bits(x)

    if nblocks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(_threads(), nblocks)) as ex:
            list(ex.map(fill, range(nblocks)))
    return out


@dataclass
class LabelDraw:
    labels: np.ndarray        # int32 [N], with ignore_index holes
    spike_rows: np.ndarray    # int64 rows that got a +spike on their (pre-ignore) label column
    spike_cols: np.ndarray    # int32 label columns of those rows
    ignored_rows: np.ndarray  # int64
    doc_starts: np.ndarray    # int64, first position of each packed document (empty if none)


def draw_labels(w: Workload, seed: int = 0) -> LabelDraw:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.wid, _LABEL_STREAM])))
    labels = g.integers(0, w.v, size=w.n, dtype=np.int32)
    spike_rows = np.empty(0, dtype=np.int64)
    if w.spike_frac > 0:
        k = int(round(w.spike_frac * w.n))
        spike_rows = np.sort(g.choice(w.n, size=k, replace=False)).astype(np.int64)
    spike_cols = labels[spike_rows].copy()
    ignored = np.empty(0, dtype=np.int64)
    if w.ignore_frac > 0:
        k = int(round(w.ignore_frac * w.n))
        ignored = np.sort(g.choice(w.n, size=k, replace=False)).astype(np.int64)
        labels[ignored] = IGNORE_INDEX
    starts = np.empty(0, dtype=np.int64)
    if w.documents > 0:
        cuts = np.sort(g.choice(np.arange(1, w.n), size=w.documents - 1, replace=False))
        starts = np.concatenate([[0], cuts]).astype(np.int64)
        labels[starts] = IGNORE_INDEX
        ignored = np.union1d(ignored, starts)
    return LabelDraw(labels, spike_rows, spike_cols, ignored, starts)


@dataclass
class CEInputs:
    logits: np.ndarray   # uint16 bf16 bits [N, V]
    labels: np.ndarray   # int32 [N]
    draw: LabelDraw


@dataclass
class FLCEInputs:
    hidden: np.ndarray   # uint16 bf16 bits [N, H]
    weight: np.ndarray   # uint16 bf16 bits [V, H]
    bias: np.ndarray | None  # float32 [V]
    labels: np.ndarray   # int32 [N]
    draw: LabelDraw


def make_ce_inputs(w: Workload, seed: int = 0) -> CEInputs:
    assert w.kind == "ce"
    d = draw_labels(w, seed)
    spikes = (d.spike_rows, d.spike_cols, w.spike) if w.spike_frac > 0 else None
    logits = normal_bf16(seed, w.wid, _T_LOGITS, w.n, w.v, w.logit_sigma, spikes)
    return CEInputs(logits, d.labels, d)


def make_flce_inputs(w: Workload, seed: int = 0) -> FLCEInputs:
    assert w.kind == "flce"
    d = draw_labels(w, seed)
    hidden = normal_bf16(seed, w.wid, _T_HIDDEN, w.n, w.h, w.hidden_sigma)
    weight = normal_bf16(seed, w.wid, _T_WEIGHT, w.v, w.h, w.weight_sigma)
    bias = None
    if w.bias_sigma > 0:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.wid, _T_BIAS, 0])))
        bias = (g.standard_normal(w.v, dtype=np.float32) * np.float32(w.bias_sigma)).astype(np.float32)
    return FLCEInputs(hidden, weight, bias, d.labels, d)


def random_ce(n: int, v: int, sigma: float = 2.0, ignore_frac: float = 0.1, seed: int = 0,
              wid: int = 1000) -> CEInputs:
    """Ad-hoc CE input of any shape (tests of edge shapes), same recipe as the workloads."""
    w = Workload(f"ce_{n}x{v}", wid, "ce", n=n, v=v, chunk_size=max(1, n),
                 logit_sigma=sigma, ignore_frac=ignore_frac)
    return make_ce_inputs(w, seed)


def random_flce(n: int, h: int, v: int, weight_sigma: float = 0.05, bias: bool = False,
                ignore_frac: float = 0.05, seed: int = 0, wid: int = 2000) -> FLCEInputs:
    w = Workload(f"flce_{n}x{h}x{v}", wid, "flce", n=n, h=h, v=v, chunk_size=max(1, n),
                 hidden_sigma=1.0, weight_sigma=weight_sigma,
                 bias_sigma=0.01 if bias else 0.0, ignore_frac=ignore_frac)
    return make_flce_inputs(w, seed)
