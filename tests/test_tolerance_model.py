"""CPU model of the rounding the HIP path introduces, at the workloads' statistics.

These tests re-derive the tolerance readings rather than trusting them: they take exact fp64
gradients (from plain matrix products of the same synthetic inputs), apply only the roundings
the GPU design performs, and measure the error against the stated bars. Nothing here calls the
GPU path; the oracle is used for the CE row values only.

Fused linear CE (rel 1e-4 on the fp32 grad_weight, read normwise): the gradient products take
the probabilities P as a bf16 operand; the design keeps the one-hot term and the scale g/T out
of that operand (applied in fp32). The normwise error of grad_weight then scales like
2^-8 · sqrt(Σ_v p_v^2 / T) per row, which depends on V and on the spread of the logits but not
on N or H, so the model keeps V and the logit standard deviation of each workload and shrinks
N and H. Alternative encodings (the scale or the one-hot inside the bf16 operand) are
simulated too, to show the choice matters: they fail the bar. Rows a trained model predicts
well (a large label probability) are modelled as well: there the label element's own bf16
rounding is as large as the whole label gradient 1 − p_y unless its residual is applied in
fp32 with the one-hot term.

Chunked CE (every gradient element within one bf16 ulp of the exact value): the kernel
computes exp in fp32, scales in fp32 and rounds once to bf16 (nearest even); the model does
the same in numpy float32 and measures the error in ulps.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import (IGNORE_INDEX, Workload, WORKLOADS, draw_labels, make_ce_inputs,
                       normal_bf16)

from _helpers import bf16_ulp, normwise_rel


def to_bf16(x):
    """fp64 → fp32 → bf16 (nearest even), the GPU's conversion chain, back as fp64."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def model_inputs(name, n, h, seed=0, peaked=0.0):
    """The workload's vocabulary size, logit spread, weight scale, bias and ignore fraction at
    n rows and h hidden columns: the hidden values are scaled by sqrt(H / h) so that h·w keeps
    the workload's spread while the weight (and with it grad_hidden) keeps its scale.
    peaked > 0 moves 30% of the hidden rows towards their label's weight row so that the
    label logit rises by `peaked` (rows a trained model predicts well)."""
    w = WORKLOADS[name]
    m = Workload(f"model_{name}", 900 + w.wid, "flce", n=n, h=h, v=w.v, chunk_size=n,
                 hidden_sigma=float(np.sqrt(w.h / h)), weight_sigma=w.weight_sigma,
                 bias_sigma=w.bias_sigma, ignore_frac=w.ignore_frac)
    hid = oracle.bf16_bits_to_f64(normal_bf16(seed, m.wid, 1, n, h, m.hidden_sigma))
    wt = oracle.bf16_bits_to_f64(normal_bf16(seed, m.wid, 2, w.v, h, w.weight_sigma))
    bias = None
    if w.bias_sigma > 0:
        g = np.random.default_rng(seed)
        bias = g.normal(0.0, w.bias_sigma, w.v).astype(np.float32).astype(np.float64)
    labels = draw_labels(m, seed).labels
    if peaked > 0:
        g = np.random.default_rng(seed + 1)
        rows = g.choice(np.nonzero(labels != IGNORE_INDEX)[0], int(0.3 * n), replace=False)
        wy = wt[labels[rows]]
        hid[rows] += peaked * wy / (wy * wy).sum(axis=1, keepdims=True)
        hid = to_bf16(hid)
    return hid, wt, bias, labels


def gradient_errors(hid, wt, bias, labels, encoding, tile=256):
    """Normwise grad_weight error, normwise and largest T·|Δ| grad_hidden error of one operand
    encoding against the exact fp64 gradients (T = labelled rows, g = 1)."""
    z = hid @ wt.T + (0.0 if bias is None else bias)
    ok = labels != IGNORE_INDEX
    t = int(ok.sum())
    s = 1.0 / t
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    p = np.exp(z - lse)
    p[~ok] = 0.0
    y = np.zeros_like(p)
    rows = np.nonzero(ok)[0]
    y[rows, labels[rows]] = 1.0
    exact_w = s * ((p - y).T @ hid)
    exact_h = s * ((p - y) @ wt)
    if encoding == "bf16(P), one-hot and g/T in fp32":
        q = to_bf16(p)
        got_w = s * (q.T @ hid) - s * (y.T @ hid)
        got_h = to_bf16(s * (q @ wt - y @ wt))
    elif encoding == "bf16(P) from fp16 shifted logits":
        v = z.shape[1]
        mt = np.empty_like(z)
        for c0 in range(0, v, tile):  # each row's maximum over its 256-column tile
            mt[:, c0:c0 + tile] = z[:, c0:c0 + tile].max(axis=1, keepdims=True)
        d = (z - mt).astype(np.float32).astype(np.float16).astype(np.float64)
        q = to_bf16(np.where(ok[:, None], np.exp(d + mt - lse), 0.0))
        got_w = s * (q.T @ hid) - s * (y.T @ hid)
        got_h = to_bf16(s * (q @ wt - y @ wt))
    elif encoding == "bf16(P), label residual and one-hot in fp32":
        q = to_bf16(p)
        # the label element's rounding residual p_y − bf16(p_y) joins the exact one-hot term
        res = np.zeros_like(p)
        res[rows, labels[rows]] = p[rows, labels[rows]] - q[rows, labels[rows]]
        got_w = s * (q.T @ hid) - s * ((y - res).T @ hid)
        got_h = to_bf16(s * (q @ wt - (y - res) @ wt))
    elif encoding == "fp16 shifted logits, label residual in fp32":
        v = z.shape[1]
        mt = np.empty_like(z)
        for c0 in range(0, v, tile):
            mt[:, c0:c0 + tile] = z[:, c0:c0 + tile].max(axis=1, keepdims=True)
        d = (z - mt).astype(np.float32).astype(np.float16).astype(np.float64)
        q = to_bf16(np.where(ok[:, None], np.exp(d + mt - lse), 0.0))
        res = np.zeros_like(p)  # the exact label probability comes from the fp32 label logit
        res[rows, labels[rows]] = p[rows, labels[rows]] - q[rows, labels[rows]]
        got_w = s * (q.T @ hid) - s * ((y - res).T @ hid)
        got_h = to_bf16(s * (q @ wt - (y - res) @ wt))
    elif encoding == "bf16(P - Y), g/T in fp32":
        q = to_bf16(p - y)
        got_w = s * (q.T @ hid)
        got_h = to_bf16(s * (q @ wt))
    elif encoding == "bf16(g/T · (P - Y))":
        q = to_bf16(s * (p - y))
        got_w = q.T @ hid
        got_h = to_bf16(q @ wt)
    else:
        raise KeyError(encoding)
    return (normwise_rel(got_w, exact_w), normwise_rel(got_h, exact_h),
            float(np.max(np.abs(got_h - exact_h))) * t)


RESIDUAL = ("bf16(P), label residual and one-hot in fp32",
            "fp16 shifted logits, label residual in fp32")
PLAIN = ("bf16(P), one-hot and g/T in fp32", "bf16(P) from fp16 shifted logits")
INSIDE = ("bf16(P - Y), g/T in fp32", "bf16(g/T · (P - Y))")

# workload, rows and hidden columns of the model (V, the logit spread and the weight scale
# are the workload's), and the label-logit rise of the peaked rows (0: none)
MODELS = [("flce_8192x4096x128256", 256, 64, 0.0), ("flce_2048x768x32777", 512, 64, 0.0),
          ("flce_32768x8192x128256_packed", 256, 64, 0.0),
          ("flce_8192x4096x128256", 256, 64, 10.0), ("flce_2048x768x32777", 512, 64, 10.0)]


@pytest.mark.parametrize("name,n,h,peaked", MODELS)
def test_probability_operand_encodings(name, n, h, peaked):
    hid, wt, bias, labels = model_inputs(name, n, h, peaked=peaked)
    res = {e: gradient_errors(hid, wt, bias, labels, e) for e in RESIDUAL + PLAIN + INSIDE}
    for e, (ew, eh, th) in res.items():
        print(f"\n[{name} model n={n} h={h} peaked={peaked}] {e}: grad_weight normwise "
              f"{ew:.2e}, grad_hidden normwise {eh:.2e}, max T·|Δ grad_hidden| {th:.2e}")
    # the design's encodings (bf16 probabilities; the one-hot term, the label element's
    # rounding residual and g/T in fp32; with or without the fp16 shift of stored logits)
    # meet the bars with room to spare, for rows a model predicts well or badly ...
    for e in RESIDUAL:
        ew, eh, th = res[e]
        assert ew <= 0.5e-4, (e, ew)
        assert eh <= 1e-2 and th <= 1e-3, (e, eh, th)
    # ... the fp16 shift of the stored logits adds little to the bf16 rounding ...
    assert res[RESIDUAL[1]][0] <= 1.5 * res[RESIDUAL[0]][0]
    if not peaked:
        # ... at the workloads' statistics the label residual changes nothing that matters ...
        for e in PLAIN:
            assert res[e][0] <= 0.5e-4, (e, res[e][0])
    else:
        # ... but where label probabilities are large, bf16(p_y) alone carries an error
        # comparable to 1 − p_y, the whole label gradient: without the residual the
        # grad_weight bar fails, and so does the one-hot term inside the operand
        for e in PLAIN + INSIDE[:1]:
            assert res[e][0] > 1e-4, (e, res[e][0])
    if name != "flce_32768x8192x128256_packed":
        # the scale g/T inside the bf16 operand (the gradient cast to the input dtype before
        # the grad_weight product) fails too: 1/T is not a power of two
        assert res[INSIDE[1]][0] > 1e-4


def test_ce_gradient_fp32_then_bf16_is_within_one_ulp():
    """The chunked CE backward's arithmetic on rows of the [16384, 128256] workload (spiked
    and plain rows): p = exp(z − lse) in fp32, times g/T in fp32, the label element as
    −(g/T)·Σ_{v≠y} p_v in fp32, one rounding to bf16. Every element lands within one ulp of
    the exact value; in fact within half an ulp plus the fp32 noise (correct rounding except
    at near-ties)."""
    w = WORKLOADS["ce_16384x128256"]
    inp = make_ce_inputs(w, seed=0)
    lab = inp.labels
    t = int((lab != IGNORE_INDEX).sum())
    rows = np.concatenate([inp.draw.spike_rows[:48], np.arange(0, w.n, 1024)])
    rows = rows[lab[rows] != IGNORE_INDEX]
    z64 = oracle.bf16_bits_to_f64(inp.logits[rows])
    exact = oracle.ce_masked_sum(z64, lab[rows], num_label_tokens=t).grad
    coef = np.float32(1.0 / t)
    z = z64.astype(np.float32)
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True, dtype=np.float32))
    p = np.exp2((z - lse) * np.float32(np.log2(np.e))).astype(np.float32)
    g = coef * p
    idx = np.arange(rows.size)
    others = p.sum(axis=1, dtype=np.float32) - p[idx, lab[rows]]
    g[idx, lab[rows]] = -coef * others
    got = to_bf16(g)
    err_ulp = np.abs(got - exact) / bf16_ulp(exact)
    print(f"\n[{w.name}] {rows.size} rows: largest error {err_ulp.max():.3f} bf16 ulp")
    assert err_ulp.max() < 1.0
    assert err_ulp.max() <= 0.5 + 1e-2
