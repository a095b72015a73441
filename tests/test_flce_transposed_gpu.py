"""GPU parity of the fused linear CE's transposed-probability schedule (through the C ABI).

With the stored-logits schedule, a grad_weight that is overwritten (no FLCE_ACCUMULATE) and a
batch no longer than about twice the hidden width, the call keeps every row's bf16
probabilities at once, transposed: the vocabulary rows that fit in the slice at its start, the
others in the bytes of the fp32 grad_weight it is about to overwrite. grad_hidden is then one
product over all rows and grad_weight one product per vocabulary range, each a plain store.
Pᵀ is kept in 64-row panels, each token-major. The cases below reach each part of that
layout: two segments of Pᵀ, several grad_weight ranges (whole tiles and single panels), a
vocabulary that ends inside a panel, padding tokens, grad_hidden split over K with
its partials in grad_weight's bytes, all of Pᵀ in the slice, and batches of more rows than one
label sort holds. Bars as in test_flce_gpu: the oracle's loss to 1e-5, every grad_weight and
grad_hidden element to the bf16 rounding budget of the probabilities, normwise 1e-4 where the
tolerance model states it.
"""
import numpy as np
import pytest
import torch

import linear_cross_entropy_masked_amd as lce
from workloads import random_flce

from _helpers import device_to_f64, gpu_device, normwise_rel
from test_flce_gpu import check, peaked_flce, run_flce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def kernels_run(fn):
    """The names of the library kernels fn() enqueues (the library's launch timing)."""
    torch.cuda.synchronize()
    lce.lce_timing_read()
    lce.lce_timing_enable(True)
    try:
        out = fn()
        torch.cuda.synchronize()
        names = {name for name, _, _ in lce.lce_timing_read()}
    finally:
        lce.lce_timing_enable(False)
    return out, names


TRANSPOSED = "flce_probs_transposed"


@pytest.mark.parametrize("n,h,v,chunk,bias", [
    (600, 320, 3001, 128, True),    # two segments, four ranges, 88-row last chunk, padding
    (640, 512, 5000, 64, False),    # ten chunks, ranges of 9 and 6 tiles
    (64, 64, 300, 64, True),        # all of Pᵀ in the slice
    (300, 256, 9000, 64, False),    # grad_hidden split five ways, partials in grad_weight
    (130, 128, 2100, 64, True),     # split two ways, a 2-row last chunk
    (384, 192, 4099, 64, True),     # h not a multiple of 256
    (1000, 640, 5003, 256, False)])
def test_transposed_schedule_parity(dev, n, h, v, chunk, bias):
    inp = random_flce(n, h, v, weight_sigma=0.1, bias=bias, ignore_frac=0.15, seed=n + 3 * h + v)
    res, names = kernels_run(lambda: run_flce(dev, inp, chunk))
    assert TRANSPOSED in names, names
    assert "flce_to_probs" not in names
    assert res["status"] == 0
    check(inp, res)


def test_transposed_schedule_peaked_rows(dev):
    """Rows a model predicts well (p_y up to 1 − 1e-7): normwise 1e-4 on grad_weight and
    grad_bias and the elementwise budget, with the label residual applied in fp32."""
    inp = peaked_flce(600, 320, 3001, seed=11, bias=True)
    res, names = kernels_run(lambda: run_flce(dev, inp, 128))
    assert TRANSPOSED in names
    check(inp, res, normwise_gw=1e-4)
    check(inp, res)


def test_more_rows_than_one_label_sort(dev):
    """8300 rows (two label sorts for the one-hot term of grad_weight), grad_weight ranges of a
    single 64-row panel (partial tiles) because a Pᵀ row takes as many bytes as a grad_weight
    row (16640 B) and the slice holds only a few panels."""
    inp = random_flce(8300, 4160, 300, weight_sigma=0.05, bias=False, ignore_frac=0.1, seed=4)
    res, names = kernels_run(lambda: run_flce(dev, inp, 2048))
    assert TRANSPOSED in names
    assert res["status"] == 0
    check(inp, res)


def test_matches_paired_schedule(dev):
    """The same call with FLCE_ACCUMULATE into zeros takes the paired schedule (grad_weight in
    fp32 read-modify-write per two chunks, grad_hidden per chunk): the same bf16 probabilities
    summed in another order. Loss and lse agree bit for bit (same logits statistics),
    grad_weight and grad_bias to fp32 summation rounding, grad_hidden to one bf16 ulp."""
    n, h, v, chunk = 600, 320, 3001, 128
    inp = random_flce(n, h, v, weight_sigma=0.1, bias=True, ignore_frac=0.1, seed=21)
    a, names_a = kernels_run(lambda: run_flce(dev, inp, chunk))
    zeros = (np.zeros((v, h)), np.zeros(v))
    b, names_b = kernels_run(lambda: run_flce(dev, inp, chunk, accumulate_init=zeros))
    assert TRANSPOSED in names_a and TRANSPOSED not in names_b and "flce_to_probs" in names_b
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["lse"], b["lse"])
    gwa, gwb = device_to_f64(a["gw"]), device_to_f64(b["gw"])
    assert normwise_rel(gwa, gwb) <= 1e-6, normwise_rel(gwa, gwb)
    assert normwise_rel(device_to_f64(a["gb"]), device_to_f64(b["gb"])) <= 1e-6
    gha, ghb = device_to_f64(a["gh"]), device_to_f64(b["gh"])
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(ghb), 1e-30))).astype(int) - 7)
    assert np.all(np.abs(gha - ghb) <= ulp + 1e-30)


def test_caller_normaliser_upstream_grad_and_zero_count(dev):
    n, h, v, chunk = 384, 192, 4099, 64
    inp = random_flce(n, h, v, weight_sigma=0.1, bias=True, ignore_frac=0.2, seed=5)
    res, names = kernels_run(lambda: run_flce(dev, inp, chunk, count=1000, g=0.37))
    assert TRANSPOSED in names
    check(inp, res, count=1000, g=0.37)
    res0 = run_flce(dev, inp, chunk, count=0)
    assert res0["loss"] == 0.0
    assert not device_to_f64(res0["gh"]).any() and not device_to_f64(res0["gw"]).any()
    assert not device_to_f64(res0["gb"]).any()
    inp.labels[:] = -100
    res1 = run_flce(dev, inp, chunk)
    assert res1["loss"] == 0.0 and not device_to_f64(res1["gw"]).any()


def test_bitwise_repeatable(dev):
    inp = random_flce(640, 512, 5000, weight_sigma=0.1, bias=True, ignore_frac=0.1, seed=9)
    a = run_flce(dev, inp, 64)
    b = run_flce(dev, inp, 64)
    assert a["loss"] == b["loss"]
    for k in ("gh", "gw", "gb"):
        assert torch.equal(a[k], b[k]), k
