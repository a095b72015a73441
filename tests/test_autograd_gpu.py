"""GPU checks of the PyTorch autograd wrappers (through the C ABI): values against the fp64
oracle, and the autograd behaviours the masked CE loss promises (out-of-place default,
opt-in in-place gradient that aliases the logits, version bump, refused second backward,
once-differentiable backward, mask folding, reductions)."""
import numpy as np
import pytest
import torch

import linear_cross_entropy_masked_amd as lce
from linear_cross_entropy_masked_amd import autograd as ag
import oracle
from workloads import random_ce, random_flce

from _helpers import (assert_close_rel, assert_faithful_bf16, bits_to_device, device_to_f64,
                      gpu_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def leaf(bits, dev):
    return bits_to_device(bits, dev).requires_grad_(True)


@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_reduced_losses_and_grads_vs_oracle(dev, reduction):
    inp = random_ce(37, 1003, sigma=2.5, ignore_frac=0.2, seed=31)
    z = leaf(inp.logits, dev)
    lab = torch.from_numpy(inp.labels.astype(np.int64)).to(dev)
    loss = ag.masked_cross_entropy(z, lab, reduction=reduction, chunk_size=8)
    loss.backward()
    ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels,
                               num_label_tokens=1 if reduction == "sum" else None)
    assert_close_rel(float(loss.item()), ref.loss, 1e-5)
    assert_faithful_bf16(device_to_f64(z.grad), ref.grad)


def test_sum_with_num_label_tokens_and_upstream_grad(dev):
    inp = random_ce(40, 700, seed=32)
    z = leaf(inp.logits, dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    loss = ag.masked_cross_entropy(z, lab, num_label_tokens=1000)
    (2.5 * loss).backward()
    ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels,
                               num_label_tokens=1000, grad_output=2.5)
    assert_close_rel(float(loss.item()), ref.loss, 1e-5)
    assert_faithful_bf16(device_to_f64(z.grad), ref.grad)


def test_reduction_none_rows_and_per_row_upstream_grads(dev):
    inp = random_ce(2 * 3 * 5, 513, sigma=2.0, ignore_frac=0.25, seed=33)
    z = leaf(inp.logits.reshape(2, 3, 5, 513), dev)
    lab = torch.from_numpy(inp.labels.reshape(2, 3, 5)).to(dev)
    rows = ag.masked_cross_entropy(z, lab, reduction="none")
    assert rows.shape == (2, 3, 5) and rows.dtype == torch.float32
    ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels,
                               num_label_tokens=1)
    got = device_to_f64(rows).reshape(-1)
    assert np.all(np.abs(got - ref.row_loss) <= 2e-6 * np.maximum(1.0, np.abs(ref.row_loss)))
    assert not got[inp.labels == -100].any()
    g = np.random.default_rng(0).normal(size=30).astype(np.float32)
    rows.backward(torch.from_numpy(g.reshape(2, 3, 5)).to(dev))
    want = ref.grad * g.astype(np.float64)[:, None]
    assert_faithful_bf16(device_to_f64(z.grad).reshape(30, 513), want)


def test_out_of_place_default_leaves_logits(dev):
    inp = random_ce(20, 300, seed=34)
    z = leaf(inp.logits, dev)
    before = z.detach().clone()
    ag.masked_cross_entropy(z, torch.from_numpy(inp.labels).to(dev)).backward()
    assert torch.equal(z.detach().view(torch.int16), before.view(torch.int16))
    assert z.grad.data_ptr() != z.data_ptr()


def test_inplace_grad_aliases_logits_bumps_version_and_refuses_rebackward(dev):
    inp = random_ce(24, 640, seed=35)
    lab = torch.from_numpy(inp.labels).to(dev)
    ref_z = leaf(inp.logits, dev)
    ag.masked_cross_entropy(ref_z, lab).backward()

    base = leaf(inp.logits, dev)
    z = base * 1  # non-leaf logits, as an lm_head output would be
    seen = []
    z.register_hook(lambda g: seen.append(g))  # the gradient as the loss hands it on
    v0 = z._version
    loss = ag.masked_cross_entropy(z, lab, inplace_grad=True)
    loss.backward(retain_graph=True)
    assert z._version > v0
    assert seen[0].data_ptr() == z.data_ptr(), "the gradient must live in the logits storage"
    assert torch.equal(z.detach().view(torch.int16), ref_z.grad.view(torch.int16))
    assert torch.equal(base.grad.view(torch.int16), ref_z.grad.view(torch.int16))
    with pytest.raises(RuntimeError):
        loss.backward()


def test_inplace_grad_breaks_other_users_of_the_logits_loudly(dev):
    inp = random_ce(16, 256, seed=36)
    lab = torch.from_numpy(inp.labels).to(dev)
    base = leaf(inp.logits, dev)
    z = base * 1
    other = (z * z).float().sum()  # saves z itself; created first, so its backward runs last
    loss = ag.masked_cross_entropy(z, lab, inplace_grad=True) + 0 * other
    with pytest.raises(RuntimeError, match="modified by an inplace operation"):
        loss.backward()


def test_double_backward_raises(dev):
    inp = random_ce(8, 100, seed=37)
    z = leaf(inp.logits, dev)
    loss = ag.masked_cross_entropy(z, torch.from_numpy(inp.labels).to(dev))
    (g,) = torch.autograd.grad(loss, z, create_graph=True)
    with pytest.raises(RuntimeError):
        g.float().sum().backward()


def test_mask_folds_into_ignore_index(dev):
    inp = random_ce(50, 400, ignore_frac=0.0, seed=38)
    mask = np.random.default_rng(1).random(50) > 0.3
    lab = torch.from_numpy(inp.labels).to(dev)
    z1 = leaf(inp.logits, dev)
    l1 = ag.masked_cross_entropy(z1, lab, mask=torch.from_numpy(mask).to(dev), reduction="mean")
    l1.backward()
    folded = np.where(mask, inp.labels, -100).astype(np.int32)
    z2 = leaf(inp.logits, dev)
    l2 = ag.masked_cross_entropy(z2, torch.from_numpy(folded).to(dev), reduction="mean")
    l2.backward()
    assert l1.item() == l2.item()
    assert torch.equal(z1.grad.view(torch.int16), z2.grad.view(torch.int16))
    ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels,
                               mask=mask.astype(np.int64))
    assert_close_rel(float(l1.item()), ref.loss, 1e-5)


def test_module_form(dev):
    inp = random_ce(30, 257, seed=39)
    m = ag.MaskedCrossEntropy(chunk_size=4, reduction="mean")
    z = leaf(inp.logits, dev)
    loss = m(z, torch.from_numpy(inp.labels).to(dev))
    loss.backward()
    ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels)
    assert_close_rel(float(loss.item()), ref.loss, 1e-5)
    assert_faithful_bf16(device_to_f64(z.grad), ref.grad)


def _flce_leaves(inp, dev):
    hid = bits_to_device(inp.hidden, dev).requires_grad_(True)
    w = bits_to_device(inp.weight, dev).requires_grad_(True)
    b = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev).requires_grad_(True)
    return hid, w, b


@pytest.mark.parametrize("bias", [False, True])
def test_linear_ce_matches_fused_call(dev, bias):
    """The autograd function (forward = flce_fwd, backward = flce_bwd) against one fused
    call of the library with the recomputing schedule on the same inputs: loss, grad_hidden
    and grad_weight (in the weight's dtype) bitwise; grad_bias (summed in another order by the
    recomputing backward) normwise to the oracle."""
    inp = random_flce(96, 64, 1000, bias=bias, seed=40)
    hid, w, b = _flce_leaves(inp, dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    loss = ag.linear_cross_entropy(hid, w, lab, b, chunk_size=40, reduction="mean")
    loss.backward()
    l2, gh, gw, gb, _ = lce.flce_fwd_bwd(hid.detach(), w.detach(), lab,
                                         None if b is None else b.detach(), chunk_size=40,
                                         recompute=True)
    assert loss.item() == l2.item()
    assert torch.equal(hid.grad.view(torch.int16), gh.view(torch.int16))
    assert torch.equal(w.grad.view(torch.int16), gw.to(torch.bfloat16).view(torch.int16))
    ref = oracle.flce(oracle.bf16_bits_to_f64(inp.hidden), oracle.bf16_bits_to_f64(inp.weight),
                      inp.labels, None if inp.bias is None else inp.bias.astype(np.float64))
    assert_close_rel(float(loss.item()), ref.loss, 1e-5)
    if bias:
        got = device_to_f64(b.grad)
        assert np.linalg.norm(got - ref.grad_bias) <= 1e-4 * np.linalg.norm(ref.grad_bias)


@pytest.mark.parametrize("bias", [False, True])
def test_linear_ce_fp32_grad_buffer_accumulates(dev, bias):
    """weight_grad_buffer takes the fp32 weight gradient (added to what it holds); a bias that
    requires grad still gets its own gradient, not added to anything stale."""
    inp = random_flce(64, 64, 517, bias=bias, seed=41)
    hid, w, b = _flce_leaves(inp, dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    buf = torch.full(tuple(w.shape), 0.25, dtype=torch.float32, device=dev)
    loss = ag.linear_cross_entropy(hid, w, lab, b, weight_grad_buffer=buf, num_label_tokens=100)
    (3.0 * loss).backward()
    assert w.grad is None, "with a buffer the weight gradient goes only into the buffer"
    g = torch.tensor(3.0, dtype=torch.float32, device=dev)
    bd = None if b is None else b.detach()
    _, gw, _ = lce.flce_bwd(hid.detach(), w.detach(), lab,
                            lce.flce_fwd(hid.detach(), w.detach(), lab, bd,
                                         num_label_tokens=100)[1],
                            bd, num_label_tokens=100, grad_output=g, grad_hidden=False,
                            grad_bias=False)
    assert torch.allclose(buf, gw + 0.25, rtol=0, atol=1e-6)
    ref = oracle.flce(oracle.bf16_bits_to_f64(inp.hidden), oracle.bf16_bits_to_f64(inp.weight),
                      inp.labels, None if inp.bias is None else inp.bias.astype(np.float64),
                      num_label_tokens=100, grad_output=3.0)
    got = buf.double().cpu().numpy() - 0.25
    assert np.linalg.norm(got - ref.grad_weight) <= 1e-4 * np.linalg.norm(ref.grad_weight)
    if bias:
        assert b.grad is not None and b.grad.dtype == torch.float32
        gotb = device_to_f64(b.grad)
        assert np.linalg.norm(gotb - ref.grad_bias) <= 1e-4 * np.linalg.norm(ref.grad_bias)


def test_interface_aliases_vs_oracle(dev):
    """ce_chunked / flce: the sum over labelled rows divided by num_label_tokens, or by the
    number of labelled rows when it is not given."""
    inp = random_ce(45, 777, seed=60)
    z = leaf(inp.logits, dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    loss = ag.ce_chunked(z, lab, chunk_size=16)
    loss.backward()
    ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels)
    assert_close_rel(float(loss.item()), ref.loss, 1e-5)
    assert_faithful_bf16(device_to_f64(z.grad), ref.grad)
    z2 = leaf(inp.logits, dev)
    loss2 = ag.ce_chunked(z2, lab, num_label_tokens=100, inplace_grad=True)
    loss2.backward()
    ref2 = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels,
                                num_label_tokens=100)
    assert_close_rel(float(loss2.item()), ref2.loss, 1e-5)

    f = random_flce(80, 64, 500, bias=True, seed=61)
    hid, w, b = _flce_leaves(f, dev)
    loss3 = ag.flce(hid, w, torch.from_numpy(f.labels).to(dev), b, chunk_size=32)
    loss3.backward()
    ref3 = oracle.flce(oracle.bf16_bits_to_f64(f.hidden), oracle.bf16_bits_to_f64(f.weight),
                       f.labels, f.bias.astype(np.float64))
    assert_close_rel(float(loss3.item()), ref3.loss, 1e-5)
    assert np.linalg.norm(device_to_f64(b.grad) - ref3.grad_bias) <= 1e-4 * np.linalg.norm(ref3.grad_bias)
