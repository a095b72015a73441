"""Seeded random sweeps over shapes, strides, value scales, ignore fractions, normalisers and
upstream gradients, each case against the fp64 oracle (through the C ABI). The case list is
drawn once from a fixed seed, so every run checks the same cases.

The bars are the scale-free ones (the stated absolute 2e-3 on bf16 gradients assumes a small
g/T, which these cases do not keep): loss relative 1e-5; lse relative 1e-5; CE gradient
elements within one bf16 ulp of the exact value; FLCE gradients within the elementwise
budget of the bf16 probability operand; rows without a label exactly zero."""
import numpy as np
import pytest
import torch

import linear_cross_entropy_masked_amd as lce
import oracle
from workloads import random_ce, random_flce

from test_ce_gpu import assert_fused_equals_two_pass, run_ce
from test_flce_gpu import rounding_bounds, run_flce
from _helpers import (assert_close_rel, assert_faithful_bf16, device_to_f64, gpu_device,
                      normwise_rel)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def _ce_cases(k=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < k:
        n = int(rng.integers(1, 300))
        v = int(np.exp(rng.uniform(0, np.log(70000))))
        if n * v > 4_000_000:
            continue
        out.append(dict(
            n=n, v=v, ld_extra=int(rng.choice([0, 1, 3, 8])), sigma=float(rng.uniform(0.5, 6)),
            ignore=float(rng.uniform(0, 0.5)), chunk=int(rng.integers(1, n + 5)),
            count=None if rng.random() < 0.5 else int(rng.integers(0, 2 * n + 2)),
            g=None if rng.random() < 0.5 else float(rng.normal(0, 2)), seed=int(rng.integers(1 << 30))))
    return out


def _flce_cases(k=12, seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < k:
        n = int(rng.integers(1, 400))
        # half the cases take h a multiple of 64, where the recomputing schedule applies
        h = 64 * int(rng.integers(1, 6)) if rng.random() < 0.5 else 8 * int(rng.integers(1, 41))
        v = int(np.exp(rng.uniform(0, np.log(9000))))
        if n * h * v > 300_000_000:
            continue
        out.append(dict(
            n=n, h=h, v=v, chunk=int(rng.integers(1, n + 5)), bias=bool(rng.random() < 0.5),
            recompute=bool(rng.random() < 0.5), ignore=float(rng.uniform(0, 0.4)),
            count=None if rng.random() < 0.6 else int(rng.integers(1, 2 * n + 2)),
            g=None if rng.random() < 0.6 else float(rng.normal(0, 2)),
            wsig=float(rng.uniform(0.01, 0.2)), seed=int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("c", _ce_cases(), ids=lambda c: f"n{c['n']}_v{c['v']}_ld{c['ld_extra']}")
def test_ce_random_case(dev, c):
    inp = random_ce(c["n"], c["v"], sigma=c["sigma"], ignore_frac=c["ignore"], seed=c["seed"])
    ld = c["v"] + c["ld_extra"]
    loss, lse, grad, status, _ = run_ce(dev, inp.logits, inp.labels, chunk=c["chunk"],
                                        count=c["count"], g=c["g"], ld=ld)
    assert status == 0
    g = 1.0 if c["g"] is None else c["g"]
    ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels,
                               num_label_tokens=c["count"], grad_output=g)
    assert_close_rel(loss, ref.loss, 1e-5)
    got = device_to_f64(grad)
    assert_faithful_bf16(got, ref.grad)
    ok, _ = oracle.labelled_rows(inp.labels, c["v"])
    assert not got[~ok].any()
    if ok.any():
        assert np.all(np.abs(lse[ok] - ref.lse[ok]) <= 1e-5 * np.maximum(1.0, np.abs(ref.lse[ok])))
    assert_fused_equals_two_pass(dev, inp.logits, inp.labels, chunk=c["chunk"],
                                 count=c["count"], g=c["g"], ld=ld)


def _flce_paired_cases(k=10, seed=2026):
    """Shapes of the compact workspace (h a multiple of 64, chunks of 64 rows or more, usually
    several of them), where two chunks share the slice; grad_bias is asked for or not, which
    decides whether the recomputing schedule pairs chunks."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < k:
        h = 64 * int(rng.integers(1, 6))
        chunk = int(rng.integers(64, 200))
        n = int(rng.integers(chunk, 4 * chunk + 1))
        v = int(np.exp(rng.uniform(np.log(2), np.log(9000))))
        if n * h * v > 300_000_000:
            continue
        bias = bool(rng.random() < 0.5)
        out.append(dict(
            n=n, h=h, v=v, chunk=chunk, bias=bias, bias_grad=bias and bool(rng.random() < 0.5),
            recompute=bool(rng.random() < 0.5), ignore=float(rng.uniform(0, 0.4)),
            count=None if rng.random() < 0.6 else int(rng.integers(1, 2 * n + 2)),
            g=None if rng.random() < 0.6 else float(rng.normal(0, 2)),
            wsig=float(rng.uniform(0.01, 0.2)), seed=int(rng.integers(1 << 30))))
    return out


def _flce_transposed_cases(k=8, seed=2028):
    """Shapes where the stored-logits schedule keeps every row's probabilities transposed in
    grad_weight's bytes and the slice: chunks a multiple of 64, batches shorter than about
    2h, hidden widths whose grad_hidden rows hold a chunk's bookkeeping (2h >= 8 * ceil(v /
    256) + 24 with v < 9000). Each case checks that the schedule ran."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < k:
        h = 64 * int(rng.integers(3, 13))
        chunk = 64 * int(rng.integers(1, 4))
        n = int(rng.integers(chunk, int(1.8 * h) + 1))
        v = int(np.exp(rng.uniform(np.log(300), np.log(9000))))
        if n * h * v > 300_000_000:
            continue
        bias = bool(rng.random() < 0.5)
        out.append(dict(
            n=n, h=h, v=v, chunk=chunk, bias=bias, bias_grad=bias and bool(rng.random() < 0.5),
            recompute=False, ignore=float(rng.uniform(0, 0.4)),
            count=None if rng.random() < 0.6 else int(rng.integers(1, 2 * n + 2)),
            g=None if rng.random() < 0.6 else float(rng.normal(0, 2)),
            wsig=float(rng.uniform(0.01, 0.2)), seed=int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("c", _flce_cases(),
                         ids=lambda c: f"n{c['n']}_h{c['h']}_v{c['v']}_c{c['chunk']}")
def test_flce_random_case(dev, c):
    _check_flce_case(dev, c)


@pytest.mark.parametrize("c", _flce_paired_cases(),
                         ids=lambda c: f"n{c['n']}_h{c['h']}_v{c['v']}_c{c['chunk']}"
                                       f"{'_rec' if c['recompute'] else ''}"
                                       f"{'_bias' if c['bias'] else ''}{'_gb' if c['bias_grad'] else ''}")
def test_flce_random_paired_case(dev, c):
    _check_flce_case(dev, c)


@pytest.mark.parametrize("c", _flce_transposed_cases(),
                         ids=lambda c: f"n{c['n']}_h{c['h']}_v{c['v']}_c{c['chunk']}"
                                       f"{'_bias' if c['bias'] else ''}{'_gb' if c['bias_grad'] else ''}")
def test_flce_random_transposed_case(dev, c):
    torch.cuda.synchronize()
    lce.lce_timing_read()
    lce.lce_timing_enable(True)
    try:
        _check_flce_case(dev, c)
        names = {name for name, _, _ in lce.lce_timing_read()}
    finally:
        lce.lce_timing_enable(False)
    assert "flce_probs_transposed" in names, names


def _check_flce_case(dev, c):
    inp = random_flce(c["n"], c["h"], c["v"], weight_sigma=c["wsig"], bias=c["bias"],
                      ignore_frac=c["ignore"], seed=c["seed"])
    res = run_flce(dev, inp, c["chunk"], count=c["count"], g=c["g"], recompute=c["recompute"],
                   want_bias_grad=c.get("bias_grad", True))
    assert res["status"] == 0
    g = 1.0 if c["g"] is None else c["g"]
    ref = oracle.flce(inp.hidden, inp.weight, inp.labels, bias=inp.bias,
                      num_label_tokens=c["count"], grad_output=g)
    assert_close_rel(res["loss"], ref.loss, 1e-5)
    ok, _ = oracle.labelled_rows(inp.labels, c["v"])
    if ok.any():
        assert np.all(np.abs(res["lse"][ok] - ref.lse[ok]) <= 1e-5 * np.maximum(1.0, np.abs(ref.lse[ok])))
    gh, gw = device_to_f64(res["gh"]), device_to_f64(res["gw"])
    assert not gh[~ok].any()
    bw, bh = rounding_bounds(inp, ref, g)
    assert np.all(np.abs(gw - ref.grad_weight) <= bw + 1e-5 * np.abs(ref.grad_weight)
                  + 1e-7 * abs(g) * ref.scale)
    ulp_h = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(ref.grad_hidden), 1e-30))).astype(int) - 8)
    assert np.all(np.abs(gh - ref.grad_hidden) <= bh + ulp_h + 1e-6 * np.abs(ref.grad_hidden) + 1e-9)
    if res["gb"] is not None and ref.grad_bias is not None and np.any(ref.grad_bias):
        assert normwise_rel(device_to_f64(res["gb"]), ref.grad_bias) <= 1e-4
