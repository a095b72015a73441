"""GPU parity of the fused linear CE against the fp64 oracle (through the C ABI).

Bars: loss relative 1e-5; grad_hidden (bf16) absolute 2e-3 and normwise relative 1e-2;
grad_weight and grad_bias (fp32) normwise relative 1e-4; rows without a label give exactly
zero grad_hidden rows.
"""
import math

import numpy as np
import pytest
import torch

import linear_cross_entropy_masked_amd as lce
import oracle
from workloads import WORKLOADS, f32_to_bf16_bits, make_flce_inputs, random_flce

from _helpers import (assert_close_rel, bits_to_device, device_to_f64, gpu_device,
                      normwise_rel)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def run_flce(dev, inp, chunk, count=None, g=None, recompute=False, accumulate_init=None,
             want_bias_grad=True):
    hid = bits_to_device(inp.hidden, dev)
    w = bits_to_device(inp.weight, dev)
    lab = torch.from_numpy(inp.labels.astype(np.int32)).to(dev)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    gout = None if g is None else torch.tensor(g, dtype=torch.float32, device=dev)
    gw = True
    gb = bias is not None and want_bias_grad
    if accumulate_init is not None:
        gw = torch.from_numpy(accumulate_init[0].astype(np.float32)).to(dev)
        if bias is not None:
            gb = torch.from_numpy(accumulate_init[1].astype(np.float32)).to(dev)
    status = torch.full((), -1, dtype=torch.int32, device=dev)
    loss, gh, gw, gb, lse = lce.flce_fwd_bwd(
        hid, w, lab, bias, chunk_size=chunk, num_label_tokens=count, recompute=recompute,
        accumulate=accumulate_init is not None, grad_output=gout, grad_weight=gw, grad_bias=gb,
        return_lse=True, status=status)
    torch.cuda.synchronize()
    return dict(loss=float(loss.item()), gh=gh, gw=gw, gb=gb, lse=lse.cpu().numpy(),
                status=int(status.item()))


def rounding_bounds(inp, ref, g):
    """Elementwise error budget of the bf16 probability operand.

    The gradient products take P rounded to bf16 (8 significant bits, round to nearest even:
    relative error at most u = 2^-8); the one-hot term and the scale g/T stay in fp32. The
    stored-logits schedule forms P from its logits kept as fp16(z − m_t), m_t the row's
    maximum over a 256-column tile: fp16 rounding (relative 2^-11) changes the exponent by at
    most 2^-11 · (m_t − z) <= 2^-11 · (max_v z − z), a relative change of P of at most
    exp(that) − 1. So P carries relative error at most r = (1 + u) · exp(2^-11 · (max z − z)) − 1
    and, up to fp32 accumulation, |ΔdW| <= |g/T| · (r·P)ᵀ|H| and |ΔdH| <= |g/T| · (r·P)|W| plus
    the final bf16 rounding of dH (half an ulp).
    """
    h = oracle.bf16_bits_to_f64(inp.hidden)
    w = oracle.bf16_bits_to_f64(inp.weight)
    z = h @ w.T + (0.0 if inp.bias is None else inp.bias.astype(np.float64))
    p = np.exp(z - ref.lse[:, None])
    ok, _ = oracle.labelled_rows(inp.labels, w.shape[0])
    p[~ok] = 0.0
    r = (1.0 + 2.0 ** -8) * np.exp(2.0 ** -11 * (z.max(axis=1, keepdims=True) - z)) - 1.0
    rp = r * p
    c = abs(g) * ref.scale
    return c * (rp.T @ np.abs(h)), c * (rp @ np.abs(w))


def sampled_hidden_budget(inp, ref_lse, rows, g, scale, fp16_shift):
    """rounding_bounds' grad_hidden budget for the rows `rows` only (their logits alone are
    formed): |Δ dH[i]| <= |g·s| · Σ_v r_iv · P_iv · |W[v]|, with r as in rounding_bounds when
    the schedule stores fp16 shifted logits, and r = 2^-8 (+ fp32 exp rounding) when it forms
    P from the fp32 logits (the recomputing schedule)."""
    h = oracle.bf16_bits_to_f64(inp.hidden[rows])
    w = oracle.bf16_bits_to_f64(inp.weight)
    z = h @ w.T + (0.0 if inp.bias is None else inp.bias.astype(np.float64))
    p = np.exp(z - ref_lse[rows][:, None])
    ok, _ = oracle.labelled_rows(inp.labels[rows], w.shape[0])
    p[~ok] = 0.0
    if fp16_shift:
        r = (1.0 + 2.0 ** -8) * np.exp(2.0 ** -11 * (z.max(axis=1, keepdims=True) - z)) - 1.0
    else:
        r = 2.0 ** -8 + 2.0 ** -20
    return abs(g) * scale * ((r * p) @ np.abs(w))


def assert_hidden_rows(gh, ref_gh, budget, count, g=1.0):
    """The bars on grad_hidden rows at the workloads: raw abs 2e-3 (stated), normwise 1e-2,
    T·|Δ| <= 2e-3 per element (the scale-free form of the stated bar), and the elementwise
    rounding budget plus half an ulp of the final bf16 rounding and fp32 slack."""
    d = np.abs(gh - ref_gh)
    assert np.max(d, initial=0.0) <= 2e-3
    assert normwise_rel(gh, ref_gh) <= 1e-2, normwise_rel(gh, ref_gh)
    assert np.max(d, initial=0.0) * count / abs(g) <= 2e-3, np.max(d) * count / abs(g)
    half_ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(ref_gh), 1e-30))).astype(int) - 8)
    excess = d - (budget + half_ulp + 1e-6 * np.abs(ref_gh) + 1e-9)
    assert np.all(excess <= 0), (float(excess.max()), np.unravel_index(excess.argmax(), d.shape))


def stores_16bit_logits(n, h, v, chunk):
    """Whether the fused call's stored-logits schedule keeps fp16 shifted logits (two chunks
    per slice): the workspace is then exactly the fp32 [chunk, ldz] slice."""
    c = min(chunk, n) if n > 0 else 1
    return lce.flce_workspace_size(n, h, v, chunk, 0) == c * ((v + 63) // 64 * 64) * 4


def check(inp, res, count=None, g=1.0, init=None, normwise_gw=None):
    """normwise_gw: the 1e-4 normwise grad_weight bar, for the workloads whose statistics it is
    stated for; other shapes are held to the elementwise rounding budget instead."""
    ref = oracle.flce(inp.hidden, inp.weight, inp.labels, bias=inp.bias, num_label_tokens=count,
                      grad_output=g, grad_weight_init=None if init is None else init[0])
    assert_close_rel(res["loss"], ref.loss, 1e-5)
    ok, _ = oracle.labelled_rows(inp.labels, inp.weight.shape[0])
    if ok.any():
        d = np.abs(res["lse"][ok] - ref.lse[ok])
        assert np.all(d <= 1e-5 * np.maximum(1.0, np.abs(ref.lse[ok]))), d.max()
    gh = device_to_f64(res["gh"])
    assert np.max(np.abs(gh - ref.grad_hidden), initial=0.0) <= 2e-3
    assert normwise_rel(gh, ref.grad_hidden) <= 1e-2
    assert not gh[~ok].any()
    gw = device_to_f64(res["gw"])
    if normwise_gw is not None:
        assert normwise_rel(gw, ref.grad_weight) <= normwise_gw, normwise_rel(gw, ref.grad_weight)
    else:
        bw, bh = rounding_bounds(inp, ref, g)
        slack_w = 1e-5 * np.abs(ref.grad_weight) + 1e-7 * np.abs(g) * ref.scale
        assert np.all(np.abs(gw - ref.grad_weight) <= bw + slack_w), \
            np.max(np.abs(gw - ref.grad_weight) - bw)
        ulp_h = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(ref.grad_hidden), 1e-30))).astype(int) - 8)
        assert np.all(np.abs(gh - ref.grad_hidden) <= bh + ulp_h + 1e-6 * np.abs(ref.grad_hidden) + 1e-9)
    if inp.bias is not None and res["gb"] is not None:
        db_ref = ref.grad_bias if init is None else ref.grad_bias + init[1]
        assert normwise_rel(device_to_f64(res["gb"]), db_ref) <= 1e-4
    return ref


@pytest.mark.parametrize("recompute", [False, True])
def test_small_model_workload_parity(dev, recompute):
    """[2048, 768] x [32777, 768] with bias, chunk 512, both schedules: every output against
    the oracle; grad_hidden also to T·|Δ| <= 2e-3 and the elementwise rounding budget of the
    schedule's probability operand, grad_weight and grad_bias to the normwise 1e-4 bar."""
    w = WORKLOADS["flce_2048x768x32777"]
    inp = make_flce_inputs(w, seed=0)
    res = run_flce(dev, inp, w.chunk_size, recompute=recompute)
    assert res["status"] == 0
    ref = check(inp, res, normwise_gw=1e-4)
    assert ref.count == 2007
    rows = np.arange(w.n)
    budget = sampled_hidden_budget(inp, ref.lse, rows, 1.0, ref.scale,
                                   fp16_shift=stores_16bit_logits(w.n, w.h, w.v, w.chunk_size)
                                   and not recompute)
    assert_hidden_rows(device_to_f64(res["gh"]), ref.grad_hidden, budget, ref.count)
    err_w = normwise_rel(device_to_f64(res["gw"]), ref.grad_weight)
    err_b = normwise_rel(device_to_f64(res["gb"]), ref.grad_bias)
    print(f"\n[{w.name} {'recompute' if recompute else 'stored fp16'}] normwise grad_weight "
          f"error {err_w:.3e}, grad_bias {err_b:.3e}, grad_hidden "
          f"{normwise_rel(device_to_f64(res['gh']), ref.grad_hidden):.3e}")


def peaked_flce(n, h, v, seed, bias=True):
    """random_flce with the rows a trained model predicts well: half of the labelled rows are
    moved along their label's weight row so that the label logit rises by 8, 12 or 20, which
    puts p_y near 0.98, 0.999 and 1 − 1e-7 at these shapes. bf16(p_y) then carries a rounding
    error as large as the label gradient 1 − p_y itself (bf16(p_y) = 1 for the largest), so
    the label element must get its residual p_y − bf16(p_y) back in fp32."""
    inp = random_flce(n, h, v, weight_sigma=0.05, bias=bias, ignore_frac=0.05, seed=seed)
    rng = np.random.default_rng(seed + 100)
    hid = oracle.bf16_bits_to_f64(inp.hidden)
    w = oracle.bf16_bits_to_f64(inp.weight)
    ok = np.nonzero(inp.labels != -100)[0]
    rows = rng.choice(ok, ok.size // 2, replace=False)
    wy = w[inp.labels[rows]]
    rise = rng.choice([8.0, 12.0, 20.0], rows.size)[:, None]
    hid[rows] += rise * wy / (wy * wy).sum(axis=1, keepdims=True)
    inp.hidden = f32_to_bf16_bits(hid.astype(np.float32))
    return inp


@pytest.mark.parametrize("n,h,v,chunk,recompute,bias", [
    (512, 128, 3000, 128, False, True),   # two chunks per slice, stored 16-bit logits
    (600, 128, 3000, 128, False, False),  # ... and a last pair of one chunk
    (394, 64, 3000, 128, False, True),    # ... a short last chunk that starts a pair of its own
    (512, 128, 3000, 128, True, False),   # two chunks per slice, recomputing
    (300, 128, 3000, 128, True, True),    # recomputing with grad_bias (one chunk per slice)
    (300, 40, 2000, 32, False, True),     # workspace beside the slice, fp32 logits
    (300, 64, 2000, 32, True, True)])     # workspace beside the slice, recomputing
def test_peaked_rows_keep_the_label_residual(dev, n, h, v, chunk, recompute, bias):
    """Rows with label probabilities near one: grad_weight normwise to 1e-4 (2e-4 at H = 40),
    grad_bias to 1e-4, and every element of grad_weight / grad_hidden to the bf16 rounding
    budget of the probabilities. The normwise bar is what needs the label element's rounding
    residual applied in fp32 with the one-hot term: the CPU rounding model of these inputs
    (bf16 probabilities, scale and one-hot in fp32) gives 1.4e-3 to 3.1e-3 without it and
    3.8e-5 to 1.2e-4 with it (1.2e-4 at H = 40, where the non-label probabilities' own bf16
    rounding weighs more; the label gradient of a p_y ~ 1 − 1e-7 row is lost entirely
    without the residual, since bf16(p_y) = 1)."""
    inp = peaked_flce(n, h, v, seed=n + h + v, bias=bias)
    res = run_flce(dev, inp, chunk, recompute=recompute)
    assert res["status"] == 0
    check(inp, res, normwise_gw=1e-4 if h >= 64 else 2e-4)
    check(inp, res)  # the elementwise budget


def test_peaked_rows_split_calls(dev):
    """flce_fwd + flce_bwd (the backward recomputes the probabilities from the saved lse) on
    rows with label probabilities near one."""
    inp = peaked_flce(512, 128, 3000, seed=5)
    hid = bits_to_device(inp.hidden, dev)
    w = bits_to_device(inp.weight, dev)
    lab = torch.from_numpy(inp.labels.astype(np.int32)).to(dev)
    b = torch.from_numpy(inp.bias).to(dev)
    loss, lse = lce.flce_fwd(hid, w, lab, b, chunk_size=128)
    gh, gw, gb = lce.flce_bwd(hid, w, lab, lse, b, chunk_size=128)
    torch.cuda.synchronize()
    check(inp, dict(loss=float(loss.item()), gh=gh, gw=gw, gb=gb, lse=lse.cpu().numpy()),
          normwise_gw=1e-4)


@pytest.mark.parametrize("n,h,v,chunk,bias", [
    (1, 8, 1, 1, False), (37, 24, 77, 10, True), (130, 136, 1000, 64, False),
    (64, 64, 65, 64, True), (200, 72, 3001, 77, True), (5, 8, 40000, 3, False),
    (257, 264, 513, 1000, True)])
def test_ragged_shapes(dev, n, h, v, chunk, bias):
    inp = random_flce(n, h, v, weight_sigma=0.1, bias=bias, ignore_frac=0.15, seed=n + h + v)
    res = run_flce(dev, inp, chunk)
    check(inp, res)


@pytest.mark.parametrize("recompute,h", [(False, 16), (True, 64)])
def test_chunk_longer_than_label_sort(dev, recompute, h):
    """A chunk of more rows than the label sort holds in LDS (8192): the one-hot term of
    grad_weight takes the per-row pass instead of the sorted label runs."""
    inp = random_flce(9000, h, 50, weight_sigma=0.1, bias=True, ignore_frac=0.1, seed=7)
    res = run_flce(dev, inp, 9000, recompute=recompute)
    assert res["status"] == 0
    check(inp, res)


@pytest.mark.parametrize("recompute,h", [(False, 40), (True, 40), (True, 64)])
def test_accumulate_into_existing_grads(dev, recompute, h):
    inp = random_flce(90, h, 333, bias=True, seed=3)
    rng = np.random.default_rng(4)
    init = (rng.normal(0, 0.01, (333, h)), rng.normal(0, 0.01, 333))
    res = run_flce(dev, inp, 32, accumulate_init=init, recompute=recompute)
    check(inp, res, init=init)


@pytest.mark.parametrize("n,h,v,chunk,bias", [
    (300, 128, 2000, 128, True), (257, 64, 513, 100, False), (96, 192, 32777, 40, True),
    (1, 64, 1, 1, True)])
def test_recompute_matches_stored_slice(dev, n, h, v, chunk, bias):
    """The recomputing schedule (logits reduced in a first GEMM pass, recomputed into bf16
    probabilities in a second) and the stored-logits schedule reduce the same fp32 logits, so
    loss and lse agree bitwise. Where the stored schedule keeps fp32 logits (the extended
    workspace) the probabilities are the same too and grad_hidden and grad_weight agree
    bitwise; where it keeps fp16 shifted logits both are held to the oracle's rounding budget.
    grad_bias is summed in another order and is held to the oracle."""
    inp = random_flce(n, h, v, weight_sigma=0.1, bias=bias, ignore_frac=0.15, seed=n + v)
    rec = run_flce(dev, inp, chunk, recompute=True)
    std = run_flce(dev, inp, chunk)
    check(inp, rec)
    check(inp, std)
    assert rec["loss"] == std["loss"]
    assert np.array_equal(rec["lse"], std["lse"])
    if not stores_16bit_logits(n, h, v, chunk):
        assert torch.equal(rec["gh"], std["gh"])
        assert torch.equal(rec["gw"], std["gw"])


@pytest.mark.parametrize("n,chunk", [(64, 64), (128, 64), (192, 64), (200, 64), (300, 100),
                                     (513, 128)])
def test_two_chunks_per_slice(dev, n, chunk):
    """The stored-logits schedule pairs chunks: an even and an odd number of chunks, a short
    last chunk alone or as the second of a pair; with grad_bias, and with an upstream gradient
    and a caller's normaliser. Loss and lse are the recomputing schedule's bit for bit."""
    h, v = 128, 1500
    assert stores_16bit_logits(n, h, v, chunk)
    inp = random_flce(n, h, v, weight_sigma=0.2, bias=True, ignore_frac=0.1, seed=n + chunk)
    res = run_flce(dev, inp, chunk, count=n - 3, g=0.75)
    assert res["status"] == 0
    check(inp, res, count=n - 3, g=0.75)
    rec = run_flce(dev, inp, chunk, count=n - 3, g=0.75, recompute=True)
    assert res["loss"] == rec["loss"]
    assert np.array_equal(res["lse"], rec["lse"])


@pytest.mark.parametrize("n,chunk", [(64, 64), (192, 64), (200, 64), (513, 128)])
def test_two_chunks_per_slice_recompute(dev, n, chunk):
    """The recomputing schedule pairs chunks too when grad_hidden rows can hold the
    bookkeeping and no grad_bias is asked for (a bias still enters the logits): against the
    oracle, and the split forward / backward calls bit for bit."""
    h, v = 128, 1500
    inp = random_flce(n, h, v, weight_sigma=0.2, bias=True, ignore_frac=0.1, seed=3 * n + chunk)
    res = run_flce(dev, inp, chunk, count=n + 1, g=1.25, recompute=True, want_bias_grad=False)
    assert res["gb"] is None
    check(inp, res, count=n + 1, g=1.25)
    hid = bits_to_device(inp.hidden, dev)
    w = bits_to_device(inp.weight, dev)
    lab = torch.from_numpy(inp.labels.astype(np.int32)).to(dev)
    b = torch.from_numpy(inp.bias).to(dev)
    gout = torch.tensor(1.25, dtype=torch.float32, device=dev)
    loss, lse = lce.flce_fwd(hid, w, lab, b, chunk_size=chunk, num_label_tokens=n + 1)
    gh, gw, gb = lce.flce_bwd(hid, w, lab, lse, b, chunk_size=chunk, num_label_tokens=n + 1,
                              grad_output=gout, grad_bias=False)
    torch.cuda.synchronize()
    assert gb is None
    assert float(loss.item()) == res["loss"]
    assert np.array_equal(lse.cpu().numpy(), res["lse"])
    assert torch.equal(gh, res["gh"])
    assert torch.equal(gw, res["gw"])


@pytest.mark.parametrize("n,chunk", [(150, 64), (300, 128)])
def test_two_chunks_per_slice_accumulate(dev, n, chunk):
    """Paired chunks adding into existing fp32 grad_weight and grad_bias (FLCE_ACCUMULATE):
    the first grad_weight product accumulates too."""
    h, v = 192, 1100
    assert stores_16bit_logits(n, h, v, chunk)
    inp = random_flce(n, h, v, weight_sigma=0.2, bias=True, ignore_frac=0.1, seed=7 * n)
    rng = np.random.default_rng(n)
    init = (rng.normal(0, 0.01, (v, h)), rng.normal(0, 0.01, v))
    res = run_flce(dev, inp, chunk, accumulate_init=init)
    check(inp, res, init=init)


@pytest.mark.parametrize("recompute,accumulate", [(False, False), (False, True), (True, False)])
def test_two_chunks_per_slice_wide_grad_weight(dev, recompute, accumulate):
    """Pairs of 2048-row chunks: grad_weight over K = 4096 rows goes through 256 × 256 tiles
    (read-modify-write when accumulating), the short last pair (2748 rows) through the two
    256 × 128 workgroups per CU; both schedules, against the oracle element by element."""
    n, h, v, chunk = 6844, 128, 1500, 2048
    assert stores_16bit_logits(n, h, v, chunk)
    inp = random_flce(n, h, v, weight_sigma=0.2, bias=True, ignore_frac=0.1,
                      seed=4096 + 2 * int(recompute) + int(accumulate))
    init = None
    if accumulate:
        rng = np.random.default_rng(4099)
        init = (rng.normal(0, 0.01, (v, h)), rng.normal(0, 0.01, v))
    res = run_flce(dev, inp, chunk, count=n - 7, g=0.5, recompute=recompute,
                   accumulate_init=init, want_bias_grad=not recompute)
    assert res["status"] == 0
    check(inp, res, count=n - 7, g=0.5, init=init)


def test_two_chunks_per_slice_without_grad_weight(dev):
    """Paired chunks when only grad_hidden is asked for: the grad_weight product and its
    one-hot term are skipped; grad_hidden, loss and lse are the full call's."""
    n, h, v, chunk = 200, 128, 900, 64
    assert stores_16bit_logits(n, h, v, chunk)
    inp = random_flce(n, h, v, weight_sigma=0.2, ignore_frac=0.1, seed=71)
    full = run_flce(dev, inp, chunk)
    hid = bits_to_device(inp.hidden, dev)
    w = bits_to_device(inp.weight, dev)
    lab = torch.from_numpy(inp.labels.astype(np.int32)).to(dev)
    loss, gh, gw, _, lse = lce.flce_fwd_bwd(hid, w, lab, chunk_size=chunk, grad_weight=False,
                                            return_lse=True)
    torch.cuda.synchronize()
    assert gw is None
    assert float(loss.item()) == full["loss"]
    assert np.array_equal(lse.cpu().numpy(), full["lse"])
    assert torch.equal(gh, full["gh"])


def test_two_chunks_per_slice_bad_labels(dev):
    """Labels outside [0, v) (other than ignore_index) in paired chunks: flagged, treated as
    ignored, never matched as a label column by the logits epilogue."""
    n, h, v, chunk = 190, 128, 700, 64
    inp = random_flce(n, h, v, weight_sigma=0.2, bias=True, ignore_frac=0.05, seed=72)
    inp.labels[[3, 70, 150]] = [v, v + 3, -7]
    res = run_flce(dev, inp, chunk)
    assert res["status"] & lce.LCE_STATUS_BAD_LABEL
    check(inp, res)
    assert not res["gh"][torch.tensor([3, 70, 150], device=dev)].any().item()


@pytest.mark.parametrize("recompute", [False, True])
def test_one_slice_workspace_and_chunk_independent_loss(dev, recompute):
    """With h a multiple of 64 and chunks of 64 rows or more the workspace is one fp32
    [chunk, ldz] slice and nothing else: the bookkeeping sits in the slice's free halves and
    in grad_hidden rows not yet written. Loss and lse are bitwise the same on either side of
    that threshold (the loss is summed row by row in fp64). grad_weight asked for without
    grad_hidden takes the recomputing passes one chunk at a time (no grad_hidden rows to
    keep the bookkeeping of two chunks per slice): within the rounding budget of the call
    with grad_hidden."""
    n, h, v = 333, 128, 3001
    ldz = (v + 63) // 64 * 64
    flags = lce.FLCE_RECOMPUTE if recompute else 0
    for c in (64, 100, n):
        assert lce.flce_workspace_size(n, h, v, c, flags) == c * ldz * 4
    assert lce.flce_workspace_size(n, h, v, 63, flags) > 63 * ldz * 4
    inp = random_flce(n, h, v, weight_sigma=0.1, ignore_frac=0.1, seed=61)
    res = {c: run_flce(dev, inp, c, recompute=recompute) for c in (63, 64, 100, n)}
    for c, r in res.items():
        assert r["status"] == 0, c
        check(inp, r)
        assert r["loss"] == res[63]["loss"], c
        assert np.array_equal(r["lse"], res[63]["lse"]), c
    hid = bits_to_device(inp.hidden, dev)
    w = bits_to_device(inp.weight, dev)
    lab = torch.from_numpy(inp.labels.astype(np.int32)).to(dev)
    loss, gh, gw, _, _ = lce.flce_fwd_bwd(hid, w, lab, chunk_size=100, recompute=recompute,
                                          grad_hidden=False)
    torch.cuda.synchronize()
    assert gh is None
    assert float(loss.item()) == res[100]["loss"]
    check(inp, dict(res[100], gw=gw))


def test_caller_normaliser_and_upstream_grad(dev):
    inp = random_flce(150, 48, 700, bias=True, seed=5)
    res = run_flce(dev, inp, 64, count=999, g=2.5)
    check(inp, res, count=999, g=2.5)


def test_zero_count_and_all_ignored(dev):
    inp = random_flce(40, 16, 100, bias=True, seed=6)
    res = run_flce(dev, inp, 16, count=0)
    assert res["loss"] == 0.0
    assert not res["gh"].any().item() and not res["gw"].any().item() and not res["gb"].any().item()
    inp.labels[:] = -100
    res = run_flce(dev, inp, 16)
    assert res["loss"] == 0.0 and not res["gw"].any().item()


def test_empty_rows(dev):
    inp = random_flce(1, 16, 50, bias=True, seed=7)
    inp.hidden = inp.hidden[:0]
    inp.labels = inp.labels[:0]
    res = run_flce(dev, inp, 4)
    assert res["loss"] == 0.0 and not res["gw"].any().item() and not res["gb"].any().item()


def test_bad_label_flagged(dev):
    inp = random_flce(30, 16, 100, seed=8, ignore_frac=0.0)
    inp.labels[3] = 100
    res = run_flce(dev, inp, 8)
    assert res["status"] & lce.LCE_STATUS_BAD_LABEL
    check(inp, res)


@pytest.mark.parametrize("recompute,h", [(False, 96), (True, 96), (True, 128)])
def test_recompute_schedule_and_chunk_invariance(dev, recompute, h):
    inp = random_flce(300, h, 2000, bias=True, seed=9)
    res = run_flce(dev, inp, 128, recompute=recompute)
    check(inp, res)
    other = run_flce(dev, inp, 77, recompute=recompute)
    assert_close_rel(other["loss"], res["loss"], 2e-7)
    assert torch.equal(other["gh"], res["gh"])


def test_bitwise_repeatable(dev):
    inp = random_flce(260, 64, 5000, bias=True, seed=10)
    a = run_flce(dev, inp, 100)
    b = run_flce(dev, inp, 100)
    assert a["loss"] == b["loss"]
    for k in ("gh", "gw", "gb"):
        assert torch.equal(a[k], b[k])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_llama3_head_workload_sampled(dev):
    """[8192, 4096] x [128256, 4096] in the launch configuration the benchmark times, and the
    same inputs with the recomputing schedule: the full loss, every row's lse, 512 complete
    grad_hidden rows (T·|Δ| and the elementwise rounding budget) and more than 512
    grad_weight rows (every label of the first chunk, plus random vocabulary rows; normwise
    1e-4) against the oracle. Rows without a label are zero in grad_hidden everywhere."""
    w = WORKLOADS["flce_8192x4096x128256"]
    inp = make_flce_inputs(w, seed=0)
    res = {rc: run_flce(dev, inp, w.chunk_size, recompute=rc) for rc in (False, True)}
    lab = inp.labels
    ok = lab != -100
    for r in res.values():
        assert r["status"] == 0
        assert not r["gh"][torch.from_numpy(np.nonzero(~ok)[0]).to(dev)].any().item()
    rng = np.random.default_rng(1)
    hrows = np.unique(np.concatenate([[0, w.n - 1], rng.choice(w.n, 510, replace=False)]))
    first_chunk = lab[:w.chunk_size]
    wrows = np.unique(np.concatenate([[0, w.v - 1], first_chunk[first_chunk >= 0],
                                      rng.choice(w.v, 512, replace=False)]))
    assert hrows.size >= 500 and wrows.size >= 1400
    ref = oracle.flce(inp.hidden, inp.weight, lab, hidden_rows=hrows, weight_rows=wrows)
    assert ref.count == 7782
    budgets = {}
    for rc, r in res.items():
        assert_close_rel(r["loss"], ref.loss, 1e-5)
        assert np.all(np.abs(r["lse"][ok] - ref.lse[ok]) <= 1e-5 * np.abs(ref.lse[ok]))
        if rc not in budgets:
            budgets[rc] = sampled_hidden_budget(inp, ref.lse, hrows, 1.0, ref.scale,
                                                fp16_shift=not rc)
        gh = device_to_f64(r["gh"][torch.from_numpy(hrows).to(dev)])
        assert_hidden_rows(gh, ref.grad_hidden, budgets[rc], ref.count)
        gw = device_to_f64(r["gw"][torch.from_numpy(wrows).to(dev)])
        err = normwise_rel(gw, ref.grad_weight)
        assert err <= 1e-4, err
        print(f"\n[{w.name} {'recompute' if rc else 'stored fp16'}] normwise grad_weight error "
              f"over {wrows.size} rows {err:.3e}; grad_hidden over {hrows.size} rows "
              f"{normwise_rel(gh, ref.grad_hidden):.3e}, max T·|Δ| "
              f"{np.max(np.abs(gh - ref.grad_hidden)) * ref.count:.3e}")
        assert math.isfinite(r["loss"])


@pytest.mark.slow
@pytest.mark.timeout(1500)
def test_long_context_packed_workload_sampled(dev):
    """[32768, 8192] x [128256, 8192], 8 packed documents, chunk 2048, with the recomputing
    schedule: the full loss and every row's lse against the oracle, 256 grad_hidden rows
    (T·|Δ| and the elementwise rounding budget of bf16 probabilities) and grad_weight rows
    (label hits and others, normwise 1e-4) on samples; the ignored rows (each document's
    first position) are zero in grad_hidden."""
    w = WORKLOADS["flce_32768x8192x128256_packed"]
    inp = make_flce_inputs(w, seed=0)
    assert int((inp.labels == -100).sum()) == 8
    res = run_flce(dev, inp, w.chunk_size, recompute=True)
    assert res["status"] == 0
    rng = np.random.default_rng(2)
    lab = inp.labels
    ok = lab != -100
    hrows = np.unique(np.concatenate([[0, w.n - 1], inp.draw.doc_starts[1:] - 1,
                                      rng.choice(w.n, 240, replace=False)]))
    hit = np.unique(lab[lab >= 0])
    wrows = np.unique(np.concatenate([[0, w.v - 1], rng.choice(hit, 128, replace=False),
                                      rng.choice(w.v, 128, replace=False)]))
    ref = oracle.flce(inp.hidden, inp.weight, lab, hidden_rows=hrows, weight_rows=wrows)
    assert ref.count == 32760
    assert_close_rel(res["loss"], ref.loss, 1e-5)
    assert np.all(np.abs(res["lse"][ok] - ref.lse[ok]) <= 1e-5 * np.abs(ref.lse[ok]))
    gh = device_to_f64(res["gh"][torch.from_numpy(hrows).to(dev)])
    budget = sampled_hidden_budget(inp, ref.lse, hrows, 1.0, ref.scale, fp16_shift=False)
    assert_hidden_rows(gh, ref.grad_hidden, budget, ref.count)
    assert not res["gh"][torch.from_numpy(np.nonzero(~ok)[0]).to(dev)].any().item()
    gw = device_to_f64(res["gw"][torch.from_numpy(wrows).to(dev)])
    err = normwise_rel(gw, ref.grad_weight)
    assert err <= 1e-4, err
    print(f"\n[{w.name} recompute] normwise grad_weight error over {wrows.size} rows "
          f"{err:.3e}; max T·|Δ| grad_hidden {np.max(np.abs(gh - ref.grad_hidden)) * ref.count:.3e}")


@pytest.mark.parametrize("n,h,v,chunk,bias,accumulate", [
    (300, 128, 2000, 128, True, False), (257, 64, 513, 100, False, True),
    (130, 40, 1000, 64, True, False), (1, 64, 1, 1, True, False)])
def test_split_forward_backward_matches_fused(dev, n, h, v, chunk, bias, accumulate):
    """flce_fwd (loss, lse) then flce_bwd (from that lse) give the loss, lse, grad_hidden and
    grad_weight of the fused call with the recomputing schedule bit for bit, and the oracle's
    grad_bias."""
    inp = random_flce(n, h, v, weight_sigma=0.1, bias=bias, ignore_frac=0.15, seed=2 * n + v)
    rng = np.random.default_rng(11)
    init = None
    if accumulate:
        init = (rng.normal(0, 0.01, (v, h)), rng.normal(0, 0.01, v))
    fused = run_flce(dev, inp, chunk, count=n + 5, g=1.5, accumulate_init=init, recompute=True)
    hid = bits_to_device(inp.hidden, dev)
    w = bits_to_device(inp.weight, dev)
    lab = torch.from_numpy(inp.labels.astype(np.int32)).to(dev)
    b = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    gout = torch.tensor(1.5, dtype=torch.float32, device=dev)
    loss, lse = lce.flce_fwd(hid, w, lab, b, chunk_size=chunk, num_label_tokens=n + 5)
    gw = True
    gb = None
    if init is not None:
        gw = torch.from_numpy(init[0].astype(np.float32)).to(dev)
        gb = torch.from_numpy(init[1].astype(np.float32)).to(dev) if b is not None else None
    gh, gw, gb = lce.flce_bwd(hid, w, lab, lse, b, chunk_size=chunk, num_label_tokens=n + 5,
                              accumulate=init is not None, grad_output=gout, grad_weight=gw,
                              grad_bias=gb if gb is not None else None)
    torch.cuda.synchronize()
    assert float(loss.item()) == fused["loss"]
    assert np.array_equal(lse.cpu().numpy(), fused["lse"])
    assert torch.equal(gh, fused["gh"])
    assert torch.equal(gw, fused["gw"])
    split = dict(loss=float(loss.item()), gh=gh, gw=gw, gb=gb, lse=lse.cpu().numpy(), status=0)
    check(inp, split, count=n + 5, g=1.5, init=init)
