"""Pins for the fp64 oracle, each independent of the oracle's own arithmetic.

The oracle is only trusted because these checks tie it to things other than itself:
closed forms, textbook special cases, brute force in plain Python, finite differences,
torch's CPU cross-entropy/autograd in fp64, and invariants of the softmax. Each pin is chosen
so that a plausible slip in the oracle (a dropped term, a wrong sign, an index mix-up, the
wrong normaliser, a missing max shift, ignored rows left non-zero) breaks at least one of
them; ``test_planted_mistakes_are_caught`` plants such slips in the oracle and checks that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import masked_ce as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _labels(rng, n, v, ignore_frac=0.25):
    y = rng.integers(0, v, n)
    y[rng.random(n) < ignore_frac] = -100
    return y


# ---------------------------------------------------------------- decoding


def test_bf16_decode_known_patterns():
    # IEEE binary32 upper halves: sign | 8-bit exponent | 7-bit fraction.
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0000: 0.0, 0x8000: -0.0,
             0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x3C00: 2.0 ** -7}
    bits = np.array(list(cases), dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert got.tolist() == list(cases.values())


def test_bf16_decode_matches_torch():
    bits = _rng(1).integers(0, 2 ** 16, 4096).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # skip inf/NaN patterns
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)


# ---------------------------------------------------------------- CE loss pins


@pytest.mark.parametrize("v", [1, 2, 1000, 128256])
def test_uniform_logits_closed_form(v):
    # All logits equal: lse = c + ln V, so each labelled row contributes ln V and the gradient
    # is s * (1/V - onehot).
    rng = _rng(v)
    n = 8
    y = _labels(rng, n, v, 0.3)
    y[0] = 0
    z = np.full((n, v), 0.625)
    r = oracle.ce_masked_sum(z, y)
    nvalid = int((y != -100).sum())
    assert r.count == nvalid
    assert math.isclose(r.loss * nvalid, nvalid * math.log(v), rel_tol=1e-13, abs_tol=1e-13)
    for i in range(n):
        if y[i] == -100:
            assert not r.grad[i].any()
        else:
            expect = np.full(v, 1.0 / v)
            expect[y[i]] -= 1.0
            np.testing.assert_allclose(r.grad[i], expect / nvalid, rtol=1e-12, atol=1e-18)


def test_closed_form_golden_cases():
    with open(os.path.join(GOLDEN, "ce_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        z = np.array(c["logits"], dtype=np.float64)
        r = oracle.ce_masked_sum(z, np.array(c["labels"]), num_label_tokens=c.get("num_label_tokens"))
        assert math.isclose(r.loss, c["loss"], rel_tol=1e-14, abs_tol=1e-300), c["name"]
        if "grad" in c:
            np.testing.assert_allclose(r.grad, np.array(c["grad"]), rtol=1e-13, atol=1e-16)


def test_two_class_is_softplus():
    # V = 2: lse - z_y = log(1 + exp(z_other - z_y)).
    rng = _rng(2)
    z = rng.normal(0, 4, (50, 2))
    y = rng.integers(0, 2, 50)
    r = oracle.ce_masked_sum(z, y, num_label_tokens=1)
    expect = sum(math.log1p(math.exp(z[i, 1 - y[i]] - z[i, y[i]])) for i in range(50))
    assert math.isclose(r.loss, expect, rel_tol=1e-13)


def test_large_margin_gives_tiny_loss():
    y = np.array([3, 999, 0, 500])
    # margin 50: each term is log(1 + 999 e^-50) ~ 1.9e-19, below fp64 resolution of lse ~ 50
    z = np.zeros((4, 1000))
    z[np.arange(4), y] = 50.0
    r = oracle.ce_masked_sum(z, y)
    assert 0 <= r.loss < 1e-18
    # margin 20: log(1 + 999 e^-20) ~ 2.06e-6, resolved to ~1e-9 relative (ulp(20) / 2e-6)
    z = np.zeros((4, 1000))
    z[np.arange(4), y] = 20.0
    r = oracle.ce_masked_sum(z, y)
    assert math.isclose(r.loss, math.log1p(999 * math.exp(-20.0)), rel_tol=1e-8)


def test_shift_invariance_and_no_overflow():
    rng = _rng(3)
    z = rng.normal(0, 3, (16, 300))
    y = _labels(rng, 16, 300)
    a = oracle.ce_masked_sum(z, y)
    b = oracle.ce_masked_sum(z + 1000.0, y)
    c = oracle.ce_masked_sum(z - 1000.0, y)
    assert np.isfinite(b.loss) and np.isfinite(c.loss)
    assert math.isclose(a.loss, b.loss, rel_tol=1e-11)
    assert math.isclose(a.loss, c.loss, rel_tol=1e-11)
    np.testing.assert_allclose(a.grad, b.grad, rtol=1e-9, atol=1e-15)


def test_brute_force_python_loops():
    # Plain-Python definition on a tiny case: no numpy, no max shift (values are small).
    rng = _rng(4)
    n, v = 5, 4
    z = rng.normal(0, 1.5, (n, v))
    y = [2, -100, 0, 3, 1]
    t = 4
    g_out = 1.75
    loss = 0.0
    grad = [[0.0] * v for _ in range(n)]
    for i in range(n):
        if y[i] == -100:
            continue
        total = sum(math.exp(z[i][k]) for k in range(v))
        loss += math.log(total) - z[i][y[i]]
        for k in range(v):
            grad[i][k] = g_out / t * (math.exp(z[i][k]) / total - (1.0 if k == y[i] else 0.0))
    loss /= t
    r = oracle.ce_masked_sum(z, np.array(y), num_label_tokens=t, grad_output=g_out)
    assert math.isclose(r.loss, loss, rel_tol=1e-14)
    np.testing.assert_allclose(r.grad, np.array(grad), rtol=1e-12, atol=1e-17)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_torch_cross_entropy_fp64(seed):
    rng = _rng(10 + seed)
    n, v = 40, 77
    z = rng.normal(0, 2.5, (n, v))
    y = _labels(rng, n, v, 0.2)
    t = 123  # a caller-supplied normaliser different from the count
    g_out = 0.37
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(y, dtype=torch.long)
    lt = F.cross_entropy(zt, yt, ignore_index=-100, reduction="sum") / t
    (lt * g_out).backward()
    r = oracle.ce_masked_sum(z, y, num_label_tokens=t, grad_output=g_out)
    assert math.isclose(r.loss, lt.item(), rel_tol=1e-13)
    np.testing.assert_allclose(r.grad, zt.grad.numpy(), rtol=1e-11, atol=1e-17)


def test_gradient_finite_differences():
    rng = _rng(5)
    n, v = 3, 5
    z = rng.normal(0, 1, (n, v))
    y = np.array([4, -100, 1])
    r = oracle.ce_masked_sum(z, y, grad_output=1.0)
    eps = 1e-6
    fd = np.zeros_like(z)
    for i in range(n):
        for k in range(v):
            zp = z.copy(); zp[i, k] += eps
            zm = z.copy(); zm[i, k] -= eps
            fd[i, k] = (oracle.ce_masked_sum(zp, y, want_grad=False).loss
                        - oracle.ce_masked_sum(zm, y, want_grad=False).loss) / (2 * eps)
    np.testing.assert_allclose(r.grad, fd, rtol=1e-6, atol=1e-9)


def test_rows_sum_to_zero_and_ignored_rows_zero():
    rng = _rng(6)
    z = rng.normal(0, 3, (64, 1000))
    y = _labels(rng, 64, 1000)
    r = oracle.ce_masked_sum(z, y)
    valid = y != -100
    assert not r.grad[~valid].any()
    np.testing.assert_allclose(r.grad[valid].sum(axis=1), 0.0, atol=1e-16)
    assert np.all(r.row_loss[~valid] == 0) and np.all(r.row_loss[valid] > 0)


def test_zero_count_guard():
    rng = _rng(7)
    z = rng.normal(0, 1, (6, 10))
    y = np.full(6, -100)
    r = oracle.ce_masked_sum(z, y)
    assert r.count == 0 and r.loss == 0.0 and not r.grad.any()
    y2 = rng.integers(0, 10, 6)
    r2 = oracle.ce_masked_sum(z, y2, num_label_tokens=0)
    assert r2.loss == 0.0 and not r2.grad.any() and np.isfinite(r2.grad).all()


def test_mask_equals_ignoring_rows():
    rng = _rng(8)
    z = rng.normal(0, 2, (30, 50))
    y = _labels(rng, 30, 50, 0.1)
    mask = rng.random(30) < 0.7
    a = oracle.ce_masked_sum(z, y, mask=mask)
    y2 = y.copy(); y2[~mask] = -100
    b = oracle.ce_masked_sum(z, y2)
    assert a.loss == b.loss and np.array_equal(a.grad, b.grad)


def test_out_of_range_label_is_flagged_and_ignored():
    z = _rng(9).normal(0, 1, (3, 7))
    y = np.array([7, -5, 2])
    r = oracle.ce_masked_sum(z, y)
    assert r.bad_label and r.count == 1
    assert not r.grad[:2].any()


def test_blocked_bits_version_matches_dense():
    from workloads import random_ce
    inp = random_ce(300, 517, sigma=3.0, ignore_frac=0.1, seed=3)
    dense = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels)
    rows = np.array([0, 5, 299, 150])
    blk = oracle.ce_masked_sum_bits(inp.logits, inp.labels, grad_rows=rows, row_block=64)
    assert math.isclose(dense.loss, blk.loss, rel_tol=1e-15)
    np.testing.assert_array_equal(dense.grad[rows], blk.grad)


def test_blocked_bits_version_upstream_grad_and_normaliser_vs_torch():
    """The row-block reader with an upstream gradient g != 1, a caller's T different from the
    count, and a row selection that includes ignored rows: pinned to torch's fp64
    cross_entropy (sum reduction) and its autograd on the CPU, not to the dense oracle."""
    from workloads import random_ce
    inp = random_ce(300, 517, sigma=3.0, ignore_frac=0.1, seed=4)
    z = oracle.bf16_bits_to_f64(inp.logits)
    t, g_out = 777, -1.75
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(inp.labels.astype(np.int64))
    lt = F.cross_entropy(zt, yt, ignore_index=-100, reduction="sum") / t
    (lt * g_out).backward()
    ignored = np.nonzero(inp.labels == -100)[0]
    rows = np.array([0, 5, 299, 150, int(ignored[0]), int(ignored[-1])])
    blk = oracle.ce_masked_sum_bits(inp.logits, inp.labels, num_label_tokens=t,
                                    grad_output=g_out, grad_rows=rows, row_block=37)
    assert blk.count == t and blk.scale == 1.0 / t
    assert math.isclose(blk.loss, lt.item(), rel_tol=1e-13)
    np.testing.assert_allclose(blk.grad, zt.grad.numpy()[rows], rtol=1e-11, atol=1e-18)
    assert not blk.grad[-2:].any()


# ---------------------------------------------------------------- FLCE pins


def _flce_case(seed, n=64, h=32, v=77, bias=True):
    rng = _rng(seed)
    hid = rng.normal(0, 1, (n, h))
    w = rng.normal(0, 0.3, (v, h))
    b = rng.normal(0, 0.1, v) if bias else None
    y = _labels(rng, n, v, 0.15)
    return hid, w, b, y


@pytest.mark.parametrize("bias", [True, False])
def test_flce_matches_torch_autograd_fp64(bias):
    hid, w, b, y = _flce_case(20, bias=bias)
    t, g_out = 47, 1.3
    ht = torch.tensor(hid, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True) if bias else None
    logits = F.linear(ht, wt, bt)
    lt = F.cross_entropy(logits, torch.tensor(y), ignore_index=-100, reduction="sum") / t
    (lt * g_out).backward()
    r = oracle.flce(hid, w, y, bias=b, num_label_tokens=t, grad_output=g_out, row_block=16)
    assert math.isclose(r.loss, lt.item(), rel_tol=1e-13)
    np.testing.assert_allclose(r.grad_hidden, ht.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(r.grad_weight, wt.grad.numpy(), rtol=1e-10, atol=1e-14)
    if bias:
        np.testing.assert_allclose(r.grad_bias, bt.grad.numpy(), rtol=1e-10, atol=1e-14)
    else:
        assert r.grad_bias is None


def test_flce_zero_weight_closed_form():
    # W = 0, b = 0: every row is uniform, so loss = ln V, grad_hidden = 0 and
    # grad_weight[v] = s (sum_valid h / V - sum_{i: y_i = v} h_i).
    rng = _rng(21)
    n, h, v = 20, 6, 9
    hid = rng.normal(0, 1, (n, h))
    y = _labels(rng, n, v, 0.2)
    valid = y != -100
    s = 1.0 / valid.sum()
    r = oracle.flce(hid, np.zeros((v, h)), y, bias=np.zeros(v))
    assert math.isclose(r.loss, math.log(v), rel_tol=1e-14)
    assert not r.grad_hidden.any()
    expect = np.tile(hid[valid].sum(axis=0) / v, (v, 1))
    for i in np.nonzero(valid)[0]:
        expect[y[i]] -= hid[i]
    np.testing.assert_allclose(r.grad_weight, s * expect, rtol=1e-12, atol=1e-15)
    counts = np.bincount(y[valid], minlength=v)
    np.testing.assert_allclose(r.grad_bias, s * (valid.sum() / v - counts), rtol=1e-12, atol=1e-15)


def test_flce_finite_differences():
    rng = _rng(22)
    n, h, v = 3, 4, 5
    hid = rng.normal(0, 1, (n, h)); w = rng.normal(0, 0.5, (v, h)); b = rng.normal(0, 0.2, v)
    y = np.array([1, 4, -100])
    r = oracle.flce(hid, w, y, bias=b)
    eps = 1e-6

    def loss(hh, ww, bb):
        return oracle.flce(hh, ww, y, bias=bb, want_grads=False).loss

    for arr, grad in ((hid, r.grad_hidden), (w, r.grad_weight), (b, r.grad_bias)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            orig = arr[idx]
            arr[idx] = orig + eps; lp = loss(hid, w, b)
            arr[idx] = orig - eps; lm = loss(hid, w, b)
            arr[idx] = orig
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-9)


def test_flce_invariants_and_reduction_to_ce():
    hid, w, b, y = _flce_case(23, n=48, h=16, v=101)
    r = oracle.flce(hid, w, y, bias=b, row_block=7)
    np.testing.assert_allclose(r.grad_weight.sum(axis=0), 0.0, atol=1e-14)
    assert abs(r.grad_bias.sum()) < 1e-14
    ce = oracle.ce_masked_sum(hid @ w.T + b, y)
    assert math.isclose(r.loss, ce.loss, rel_tol=1e-14)


def test_flce_accumulate_and_row_selection():
    hid, w, b, y = _flce_case(24, n=30, h=8, v=40)
    init = _rng(25).normal(0, 1, (40, 8))
    full = oracle.flce(hid, w, y, bias=b)
    acc = oracle.flce(hid, w, y, bias=b, grad_weight_init=init)
    np.testing.assert_allclose(acc.grad_weight, full.grad_weight + init, rtol=1e-14, atol=1e-15)
    hr = np.array([29, 0, 7]); wr = np.array([39, 3])
    sub = oracle.flce(hid, w, y, bias=b, hidden_rows=hr, weight_rows=wr, row_block=8)
    np.testing.assert_allclose(sub.grad_hidden, full.grad_hidden[hr], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(sub.grad_weight, full.grad_weight[wr], rtol=1e-13, atol=1e-16)


def test_flce_accepts_bf16_bits():
    from workloads import random_flce
    inp = random_flce(16, 8, 21, bias=True, seed=1)
    a = oracle.flce(inp.hidden, inp.weight, inp.labels, bias=inp.bias)
    b = oracle.flce(oracle.bf16_bits_to_f64(inp.hidden), oracle.bf16_bits_to_f64(inp.weight),
                    inp.labels, bias=inp.bias.astype(np.float64))
    assert a.loss == b.loss


# ---------------------------------------------------------------- planted mistakes


def _pins_pass():
    """Run a handful of the pins above; True if all of them hold."""
    try:
        test_uniform_logits_closed_form(1000)
        test_two_class_is_softplus()
        test_shift_invariance_and_no_overflow()
        test_matches_torch_cross_entropy_fp64(0)
        test_rows_sum_to_zero_and_ignored_rows_zero()
        test_zero_count_guard()
        test_brute_force_python_loops()
    except AssertionError:
        return False
    except FloatingPointError:
        return False
    return True


def test_planted_mistakes_are_caught(monkeypatch):
    assert _pins_pass()

    def no_shift(z):
        with np.errstate(over="ignore"):
            return np.log(np.sum(np.exp(z), axis=1))

    def wrong_scale(t):
        return 1.0 / (t + 1.0) if t > 0 else 0.0

    def zero_guard_missing(t):
        return 1.0 / t if t > 0 else float("inf")

    planted = [("logsumexp_rows", no_shift), ("scale_from_count", wrong_scale),
               ("scale_from_count", zero_guard_missing)]
    for name, fn in planted:
        with monkeypatch.context() as m:
            m.setattr(om, name, fn)
            with np.errstate(all="ignore"):
                assert not _pins_pass(), f"planted mistake in {name} went unnoticed"
