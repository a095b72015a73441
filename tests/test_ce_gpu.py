"""GPU parity of the chunked masked CE kernels against the fp64 oracle (through the C ABI).

Bars (loss: relative 1e-5; every gradient element within one bf16 ulp of the exact fp64
value, which also implies the stated absolute 2e-3; ignored rows exactly zero).
"""
import math

import numpy as np
import pytest
import torch

import linear_cross_entropy_masked_amd as lce
import oracle
from workloads import WORKLOADS, make_ce_inputs, random_ce, random_flce

from _helpers import (assert_close_rel, assert_faithful_bf16, bf16_ulp, bits_to_device,
                      device_to_f64, gpu_device, oracle_ce_rows_parallel)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def run_ce(dev, bits, labels, chunk=16, count=None, inplace=True, g=None, save_lse=True, ld=None):
    n, v = bits.shape
    if ld is None or ld == v:
        logits = bits_to_device(bits, dev)
    else:  # rows ld elements apart
        buf = torch.zeros((n, ld), dtype=torch.bfloat16, device=dev)
        buf[:, :v] = bits_to_device(bits, dev)
        logits = buf[:, :v]
    lab = torch.from_numpy(labels.astype(np.int32)).to(dev)
    status = torch.full((), -1, dtype=torch.int32, device=dev)
    loss, lse = lce.ce_chunked_fwd(logits, lab, chunk_size=chunk, num_label_tokens=count,
                                   return_lse=save_lse, status=status)
    gout = None if g is None else torch.tensor(g, dtype=torch.float32, device=dev)
    if inplace:
        grad = lce.ce_chunked_bwd_inplace(logits, lab, chunk_size=chunk, num_label_tokens=count,
                                          grad_output=gout, lse=lse)
        assert grad.data_ptr() == logits.data_ptr()
    else:
        grad = lce.ce_chunked_bwd(logits, lab, chunk_size=chunk, num_label_tokens=count,
                                  grad_output=gout, lse=lse)
    torch.cuda.synchronize()
    return (float(loss.item()), None if lse is None else lse.cpu().numpy(), grad,
            int(status.item()), logits)


def check_against_oracle(bits, labels, loss, lse, grad, count=None, g=1.0):
    z = oracle.bf16_bits_to_f64(bits)
    ref = oracle.ce_masked_sum(z, labels, num_label_tokens=count, grad_output=g)
    assert_close_rel(loss, ref.loss, 1e-5)
    got = device_to_f64(grad)
    assert_faithful_bf16(got, ref.grad)
    assert np.max(np.abs(got - ref.grad), initial=0.0) <= 2e-3
    ok, _ = oracle.labelled_rows(labels, bits.shape[1])
    assert not got[~ok].any(), "rows without a label must be exactly zero"
    if lse is not None and ok.any():
        d = np.abs(lse[ok] - ref.lse[ok])
        assert np.all(d <= 2e-6 * np.maximum(1.0, np.abs(ref.lse[ok])))
        assert not lse[~ok].any()
    return ref


def test_small_workload_parity_in_place(dev):
    w = WORKLOADS["ce_64x1000"]
    inp = make_ce_inputs(w, seed=0)
    loss, lse, grad, status, _ = run_ce(dev, inp.logits, inp.labels, chunk=w.chunk_size)
    assert status == 0
    ref = check_against_oracle(inp.logits, inp.labels, loss, lse, grad)
    assert ref.count == 58


@pytest.mark.parametrize("n,v", [(1, 1), (3, 2), (5, 7), (17, 1000), (33, 32777), (6, 128256),
                                 (300, 517), (64, 8), (9, 9)])
def test_edge_shapes(dev, n, v):
    inp = random_ce(n, v, sigma=2.5, ignore_frac=0.2, seed=n * 7 + v)
    loss, lse, grad, status, _ = run_ce(dev, inp.logits, inp.labels, chunk=5)
    assert status == 0
    check_against_oracle(inp.logits, inp.labels, loss, lse, grad)


@pytest.mark.parametrize("ld_extra", [1, 3, 8, 13])
def test_row_stride_larger_than_v(dev, ld_extra):
    n, v = 21, 777
    inp = random_ce(n, v, seed=ld_extra)
    loss, lse, grad, _, _ = run_ce(dev, inp.logits, inp.labels, chunk=4, ld=v + ld_extra)
    check_against_oracle(inp.logits, inp.labels, loss, lse, grad)


def test_empty_input(dev):
    bits = np.zeros((0, 10), dtype=np.uint16)
    labels = np.zeros(0, dtype=np.int32)
    loss, lse, grad, status, _ = run_ce(dev, bits, labels, chunk=4)
    assert loss == 0.0 and grad.numel() == 0 and status == 0


def test_out_of_place_leaves_logits_and_matches_in_place(dev):
    inp = random_ce(40, 3001, seed=11)
    l1, _, g_in, _, _ = run_ce(dev, inp.logits, inp.labels, inplace=True)
    l2, _, g_out, _, logits = run_ce(dev, inp.logits, inp.labels, inplace=False)
    assert l1 == l2
    assert torch.equal(g_in, g_out)
    np.testing.assert_array_equal(
        logits.view(torch.int16).cpu().numpy().view(np.uint16), inp.logits)


@pytest.mark.parametrize("ld_extra", [1, 3])
def test_out_of_place_with_different_row_alignment(dev, ld_extra):
    """Logits rows ld = v + odd apart, gradient rows v apart: on the rows whose 16-byte phase
    differs the backward takes its scalar path (label element included)."""
    inp = random_ce(33, 1003, sigma=3.0, ignore_frac=0.2, seed=40 + ld_extra)
    loss, lse, grad, status, _ = run_ce(dev, inp.logits, inp.labels, inplace=False,
                                        ld=1003 + ld_extra, g=0.75, count=17)
    assert status == 0
    check_against_oracle(inp.logits, inp.labels, loss, lse, grad, count=17, g=0.75)


def test_recomputed_lse_matches_saved(dev):
    inp = random_ce(50, 4099, sigma=3.0, seed=12)
    _, _, g_saved, _, _ = run_ce(dev, inp.logits, inp.labels, save_lse=True)
    _, _, g_recomp, _, _ = run_ce(dev, inp.logits, inp.labels, save_lse=False)
    assert torch.equal(g_saved, g_recomp)


def test_zero_count_guard_and_all_ignored(dev):
    inp = random_ce(12, 300, seed=13, ignore_frac=0.0)
    loss, _, grad, _, _ = run_ce(dev, inp.logits, inp.labels, count=0)
    assert loss == 0.0 and not grad.any().item()
    labels = np.full(12, -100, dtype=np.int32)
    loss, _, grad, status, _ = run_ce(dev, inp.logits, labels)
    assert loss == 0.0 and not grad.any().item() and status == 0


def test_caller_normaliser_and_upstream_grad(dev):
    inp = random_ce(70, 2048, seed=14)
    loss, lse, grad, _, _ = run_ce(dev, inp.logits, inp.labels, count=1234, g=0.37)
    check_against_oracle(inp.logits, inp.labels, loss, lse, grad, count=1234, g=0.37)


def test_chunk_size_invariance(dev):
    inp = random_ce(97, 5003, sigma=3.0, seed=15)
    base = None
    for chunk in (1, 7, 16, 1000, 97, 10_000):
        loss, _, grad, _, _ = run_ce(dev, inp.logits, inp.labels, chunk=chunk)
        if base is None:
            base = (loss, grad)
        else:
            assert loss == base[0]
            assert torch.equal(grad, base[1])


def test_bitwise_repeatable(dev):
    inp = random_ce(64, 32777, sigma=3.0, seed=16)
    runs = [run_ce(dev, inp.logits, inp.labels) for _ in range(3)]
    for r in runs[1:]:
        assert r[0] == runs[0][0]
        assert torch.equal(r[2], runs[0][2])


def test_out_of_range_labels_flagged_and_ignored(dev):
    inp = random_ce(10, 100, seed=17, ignore_frac=0.0)
    labels = inp.labels.copy()
    labels[2] = 100
    labels[5] = -7
    loss, lse, grad, status, _ = run_ce(dev, inp.logits, labels)
    assert status & lce.LCE_STATUS_BAD_LABEL
    ref = check_against_oracle(inp.logits, labels, loss, lse, grad)
    assert ref.bad_label and ref.count == 8


def all_rows_invariants(grad, labels, count, rows_per_copy=512):
    """Every row of a [n, v] bf16 gradient, checked on the host block by block: rows without
    a label exactly zero; for a labelled row the exact gradient sums to zero (softmax minus
    one-hot), so |Σ_v g_v| can only be the rounding of its elements: at most Σ_v ½ ulp(g_v)
    (round to nearest) plus fp32 slack. (A fixed bar such as |Σ_v T·g| <= 4e-3 is not a
    bound: rounding the oracle's exact gradient to nearest already reaches 4.3e-3 at the
    [16384, 128256] statistics.) Returns the largest |Σ_v T·g| and the largest ratio of
    |Σ_v g| to its bound."""
    n = grad.shape[0]
    ok = labels != -100
    worst = ratio = 0.0
    for r0 in range(0, n, rows_per_copy):
        r1 = min(n, r0 + rows_per_copy)
        blk = grad[r0:r1].view(torch.int16).cpu().numpy()
        g = oracle.bf16_bits_to_f64(blk)
        okb = ok[r0:r1]
        assert not g[~okb].any(), f"a row without a label is nonzero in rows {r0}..{r1}"
        gl = g[okb]
        if not gl.size:
            continue
        sums = np.abs(gl.sum(axis=1))
        bound = 0.5 * bf16_ulp(gl).sum(axis=1) + 2.0 ** -20 * np.abs(gl).sum(axis=1)
        bad = sums > bound
        assert not bad.any(), (r0 + np.nonzero(okb)[0][np.argmax(bad)], sums.max(), bound.min())
        worst = max(worst, float(sums.max()) * count)
        ratio = max(ratio, float((sums / np.maximum(bound, 1e-300)).max()))
    return worst, ratio


@pytest.mark.timeout(600)
def test_large_vocab_workload_full_size(dev):
    """[16384, 128256] in the launch configuration the benchmark times: full loss and every
    row's lse against the oracle; every row of the gradient checked on the host (zero rows
    without a label, rows of labelled tokens summing to zero within rounding); 512 and more
    complete gradient rows (random, spiked, ignored, first and last) within one bf16 ulp of
    the oracle, element by element."""
    w = WORKLOADS["ce_16384x128256"]
    inp = make_ce_inputs(w, seed=0)
    labels = inp.labels
    count = int((labels != -100).sum())
    assert count == 15565
    loss, lse, grad, status, _ = run_ce(dev, inp.logits, labels, chunk=w.chunk_size)
    assert status == 0
    row_loss, ref_lse = oracle_ce_rows_parallel(inp.logits, labels, count)
    assert_close_rel(loss, math.fsum(row_loss) / count, 1e-5)
    ok = labels != -100
    assert np.all(np.abs(lse[ok] - ref_lse[ok]) <= 2e-6 * np.abs(ref_lse[ok]))
    assert not lse[~ok].any()
    worst, ratio = all_rows_invariants(grad, labels, count)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([
        [0, w.n - 1], rng.choice(w.n, 512, replace=False), inp.draw.spike_rows[:32],
        inp.draw.ignored_rows[:16]]))
    assert rows.size >= 512
    got = device_to_f64(grad[torch.from_numpy(rows).to(dev)])
    for k, r in enumerate(rows):
        z = oracle.bf16_bits_to_f64(inp.logits[r:r + 1])
        one = oracle.ce_masked_sum(z, labels[r:r + 1], num_label_tokens=count)
        assert_faithful_bf16(got[k:k + 1], one.grad, what=f"grad row {r}")
        if labels[r] == -100:
            assert not got[k].any()
    print(f"\n[{w.name}] max |sum_v T*g| over all labelled rows {worst:.3e} "
          f"(largest fraction of its rounding bound {ratio:.3f}); {rows.size} rows within one "
          f"bf16 ulp")


# ---- single pass (ce_chunked_fwd_bwd_inplace) --------------------------------------------

def run_fused(dev, bits, labels, chunk=16, count=None, g=None, ld=None, return_lse=True):
    n, v = bits.shape
    if ld is None or ld == v:
        logits = bits_to_device(bits, dev)
    else:
        buf = torch.zeros((n, ld), dtype=torch.bfloat16, device=dev)
        buf[:, :v] = bits_to_device(bits, dev)
        logits = buf[:, :v]
    lab = torch.from_numpy(labels.astype(np.int32)).to(dev)
    status = torch.full((), -1, dtype=torch.int32, device=dev)
    gout = None if g is None else torch.tensor(g, dtype=torch.float32, device=dev)
    loss, lse = lce.ce_chunked_fwd_bwd_inplace(logits, lab, chunk_size=chunk,
                                               num_label_tokens=count, grad_output=gout,
                                               return_lse=return_lse, status=status)
    torch.cuda.synchronize()
    return loss, lse, logits, int(status.item())


def assert_fused_equals_two_pass(dev, bits, labels, chunk=16, count=None, g=None, ld=None):
    loss_a, lse_a, grad_a, st_a, _ = run_ce(dev, bits, labels, chunk=chunk, count=count, g=g,
                                            ld=ld)
    loss_b, lse_b, grad_b, st_b = run_fused(dev, bits, labels, chunk=chunk, count=count, g=g,
                                            ld=ld)
    assert st_a == st_b
    assert np.float32(loss_a).tobytes() == loss_b.cpu().numpy().tobytes()
    assert np.array_equal(lse_a.view(np.uint32), lse_b.cpu().numpy().view(np.uint32))
    assert torch.equal(grad_a.view(torch.int16), grad_b.view(torch.int16)), "gradient bits differ"
    return loss_b, lse_b, grad_b, st_b


# rows per lane-vector count: v/8 <= 4096 (4 vectors per lane), <= 8192 (8), <= 16384 (16),
# and past it (the two passes inside the call); ld_extra shifts each row's alignment. The
# cases with more rows than the GPU has CUs keep several rows per CU in flight, ignored rows
# among them.
@pytest.mark.parametrize("n,v,ld_extra", [
    (1, 1, 0), (3, 7, 0), (64, 1000, 0), (17, 1000, 3), (33, 32777, 0), (5, 32775, 1),
    (9, 40000, 5), (5, 65543, 0), (7, 70001, 1), (6, 128256, 0), (4, 131079, 0),
    (3, 131080, 2), (3, 140000, 0), (600, 1000, 0), (1100, 24, 0), (520, 32776, 8),
    (300, 65544, 0), (290, 128256, 0), (777, 8192, 0)])
def test_fused_bitwise_equals_two_pass(dev, n, v, ld_extra):
    inp = random_ce(n, v, sigma=2.5, ignore_frac=0.2, seed=n * 13 + v + ld_extra)
    assert_fused_equals_two_pass(dev, inp.logits, inp.labels, ld=v + ld_extra)


def test_fused_small_workload_vs_oracle(dev):
    w = WORKLOADS["ce_64x1000"]
    inp = make_ce_inputs(w, seed=0)
    loss, lse, grad, status = run_fused(dev, inp.logits, inp.labels, chunk=w.chunk_size)
    assert status == 0
    ref = check_against_oracle(inp.logits, inp.labels, float(loss.item()), lse.cpu().numpy(),
                               grad)
    assert ref.count == 58


def test_fused_zero_count_all_ignored_and_upstream_grad(dev):
    inp = random_ce(12, 300, seed=21, ignore_frac=0.0)
    loss, lse, grad, _ = run_fused(dev, inp.logits, inp.labels, count=0)
    assert float(loss.item()) == 0.0 and not grad.float().abs().sum().item()
    assert np.all(lse.cpu().numpy() != 0)  # lse still reported for labelled rows
    labels = np.full_like(inp.labels, -100)
    loss, lse, grad, _ = run_fused(dev, inp.logits, labels)
    assert float(loss.item()) == 0.0 and not grad.float().abs().sum().item()
    assert not lse.cpu().numpy().any()
    inp = random_ce(70, 2048, seed=22)
    assert_fused_equals_two_pass(dev, inp.logits, inp.labels, count=1000, g=2.5)
    loss, lse, grad, _ = run_fused(dev, inp.logits, inp.labels, count=1000, g=2.5)
    check_against_oracle(inp.logits, inp.labels, float(loss.item()), lse.cpu().numpy(), grad,
                         count=1000, g=2.5)


def test_fused_row_loop_zero_count_and_upstream_grad(dev):
    """More rows than CUs: T = 0 (lse and loss terms kept, every gradient element written as
    +0), an all-ignored batch, and a caller's T and upstream gradient, bitwise the two
    passes."""
    inp = random_ce(700, 1000, seed=31, ignore_frac=0.1)
    loss, lse, grad, _ = run_fused(dev, inp.logits, inp.labels, count=0)
    assert float(loss.item()) == 0.0
    assert not grad.view(torch.int16).any().item(), "T = 0 must write +0 everywhere"
    assert np.all(lse.cpu().numpy()[inp.labels != -100] != 0)
    labels = np.full_like(inp.labels, -100)
    loss, lse, grad, _ = run_fused(dev, inp.logits, labels)
    assert float(loss.item()) == 0.0 and not grad.view(torch.int16).any().item()
    assert not lse.cpu().numpy().any()
    assert_fused_equals_two_pass(dev, inp.logits, inp.labels, count=5000, g=0.75)


def test_fused_bad_labels_flagged_and_empty(dev):
    inp = random_ce(10, 100, seed=23, ignore_frac=0.0)
    labels = inp.labels.copy()
    labels[2] = 100
    labels[5] = -7
    _, _, _, status = assert_fused_equals_two_pass(dev, inp.logits, labels)
    assert status & lce.LCE_STATUS_BAD_LABEL
    empty = torch.empty((0, 50), dtype=torch.bfloat16, device=dev)
    loss, lse = lce.ce_chunked_fwd_bwd_inplace(
        empty, torch.empty(0, dtype=torch.int32, device=dev), return_lse=True)
    assert float(loss.item()) == 0.0 and lse.numel() == 0


@pytest.mark.timeout(600)
def test_fused_large_vocab_workload_full_size(dev):
    """[16384, 128256], the launch configuration the benchmark times: bitwise the two passes
    (whose values the full-size two-pass test pins to the oracle)."""
    w = WORKLOADS["ce_16384x128256"]
    inp = make_ce_inputs(w, seed=0)
    _, _, grad, status = assert_fused_equals_two_pass(dev, inp.logits, inp.labels,
                                                      chunk=w.chunk_size)
    assert status == 0
    all_rows_invariants(grad, inp.labels, int((inp.labels != -100).sum()))


def test_binding_rejects_short_or_strided_lse(dev):
    """The CE backward bindings pass lse to the kernels as a plain [n] array: a shorter or
    strided tensor is refused before any launch."""
    inp = random_ce(8, 100, seed=30)
    logits = bits_to_device(inp.logits, dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    short = torch.zeros(7, dtype=torch.float32, device=dev)
    strided = torch.zeros(16, dtype=torch.float32, device=dev)[::2]
    grad_rows = torch.ones(8, dtype=torch.float32, device=dev)
    for lse in (short, strided):
        with pytest.raises(ValueError):
            lce.ce_chunked_bwd(logits, lab, lse=lse)
        with pytest.raises(ValueError):
            lce.ce_chunked_bwd_inplace(logits, lab, lse=lse)
        with pytest.raises(ValueError):
            lce.ce_rows_bwd(logits, lab, grad_rows, lse=lse)


def test_int64_labels_outside_int32_are_flagged_not_wrapped(dev):
    """An int64 label such as 2**32 + 5 is not class 5: the binding keeps it out of range, so
    the row is unlabelled and the status bit is set (both layers)."""
    inp = random_ce(10, 100, seed=31, ignore_frac=0.0)
    lab64 = torch.from_numpy(inp.labels.astype(np.int64))
    lab64[3] = 2 ** 32 + 5
    lab64[6] = -(2 ** 33)
    ref_labels = inp.labels.copy()
    ref_labels[3] = 100   # any out-of-range label: the oracle flags it and ignores the row
    ref_labels[6] = -7
    for ignore_index in (-100, -1):
        status = torch.full((), -1, dtype=torch.int32, device=dev)
        logits = bits_to_device(inp.logits, dev)
        loss, lse = lce.ce_chunked_fwd(logits, lab64.to(dev), ignore_index=ignore_index,
                                       status=status)
        torch.cuda.synchronize()
        assert int(status.item()) & lce.LCE_STATUS_BAD_LABEL
        ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), ref_labels,
                                   ignore_index=ignore_index)
        assert ref.count == 8
        assert_close_rel(float(loss.item()), ref.loss, 1e-5)
    f = random_flce(12, 16, 50, seed=32, ignore_frac=0.0)
    fl = torch.from_numpy(f.labels.astype(np.int64))
    fl[2] = 2 ** 31
    status = torch.full((), -1, dtype=torch.int32, device=dev)
    loss, gh, _, _, _ = lce.flce_fwd_bwd(bits_to_device(f.hidden, dev), bits_to_device(f.weight, dev),
                                         fl.to(dev), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & lce.LCE_STATUS_BAD_LABEL
    assert not gh[2].any().item()
    ref_l = f.labels.copy()
    ref_l[2] = 50
    r = oracle.flce(f.hidden, f.weight, ref_l)
    assert_close_rel(float(loss.item()), r.loss, 1e-5)
