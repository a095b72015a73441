"""The allocation-free CE step (ce_chunked_fwd_bwd_inplace_noalloc) through the C ABI: bit for
bit the results of the workspace-taking ce_chunked_fwd_bwd_inplace on the same inputs, call
after call, with the second call smaller than the first (the static scratch keeps the first
call's contents), and within the oracle's bars."""
import ctypes

import numpy as np
import pytest
import torch

import linear_cross_entropy_masked_amd as lce
import oracle
from workloads import random_ce

from _helpers import assert_close_rel, assert_faithful_bf16, device_to_f64, gpu_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def strided_logits(bits, ld, dev):
    n, v = bits.shape
    buf = torch.zeros((n, ld), dtype=torch.bfloat16, device=dev)
    buf[:, :v] = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    return buf


def run_both(dev, inp, ld, count, g):
    """The same step through both entry points on identical inputs; returns their outputs."""
    n, v = inp.logits.shape
    lib = lce.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    lab = torch.from_numpy(inp.labels).to(dev)
    gout = torch.tensor(g, dtype=torch.float32, device=dev)
    out = {}
    for name in ("noalloc", "workspace"):
        buf = strided_logits(inp.logits, ld, dev)
        loss = torch.full((), -1.0, dtype=torch.float32, device=dev)
        lse = torch.full((n,), -1.0, dtype=torch.float32, device=dev)
        status = torch.full((), -1, dtype=torch.int32, device=dev)
        if name == "noalloc":
            rc = lib.ce_chunked_fwd_bwd_inplace_noalloc(
                ctypes.c_void_p(buf.data_ptr()), n, v, ld, ctypes.c_void_p(lab.data_ptr()), -100,
                256, count, ctypes.c_void_p(gout.data_ptr()), ctypes.c_void_p(loss.data_ptr()),
                ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(status.data_ptr()), stream)
        else:
            nbytes = lce.ce_chunked_workspace_size(n, v, 256)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            rc = lib.ce_chunked_fwd_bwd_inplace(
                ctypes.c_void_p(buf.data_ptr()), n, v, ld, ctypes.c_void_p(lab.data_ptr()), -100,
                256, count, ctypes.c_void_p(gout.data_ptr()), ctypes.c_void_p(loss.data_ptr()),
                ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(status.data_ptr()),
                ctypes.c_void_p(ws.data_ptr()), nbytes, stream)
        assert rc == 0, (name, rc, lce.lce_status_str(rc))
        torch.cuda.synchronize()
        out[name] = (loss, lse, buf, status)
    return out


def assert_same(out):
    a, b = out["noalloc"], out["workspace"]
    assert a[0].view(torch.int32).item() == b[0].view(torch.int32).item(), (a[0], b[0])
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
    assert torch.equal(a[2].view(torch.int16), b[2].view(torch.int16))
    assert a[3].item() == b[3].item()


@pytest.mark.parametrize("first,second", [((2000, 32777, 5), (300, 1000, 0)),
                                          ((700, 5003, 3), (9, 140000, 8))])
def test_noalloc_step_equals_workspace_step_twice(dev, first, second):
    """Two calls in a row, the second with fewer rows (one pair also switches to rows too long
    for registers, which take the two-pass path), each bit for bit the workspace call's and
    within the oracle's bars."""
    for k, (n, v, pad) in enumerate((first, second)):
        inp = random_ce(n, v, sigma=3.0, ignore_frac=0.15, seed=100 + 7 * k + n)
        count = n + 11 if k == 0 else -1
        g = 0.5 if k == 0 else 1.25
        out = run_both(dev, inp, v + pad, count, g)
        assert_same(out)
        loss, lse, buf, status = out["noalloc"]
        assert status.item() == 0
        ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels,
                                   num_label_tokens=None if count < 0 else count, grad_output=g)
        assert_close_rel(float(loss.item()), ref.loss, 1e-5)
        assert_faithful_bf16(device_to_f64(buf[:, :v]), ref.grad)
        ok = inp.labels != -100
        got = lse.cpu().numpy()
        assert np.all(np.abs(got[ok] - ref.lse[ok]) <= 2e-6 * np.maximum(1.0, np.abs(ref.lse[ok])))


def test_noalloc_binding_and_scratch_limit(dev):
    inp = random_ce(64, 1000, seed=7)
    logits = strided_logits(inp.logits, 1000, dev)
    twin = logits.clone()
    lab = torch.from_numpy(inp.labels).to(dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    l1, _ = lce.ce_chunked_fwd_bwd_inplace_noalloc(logits, lab, loss=loss)
    l2, _ = lce.ce_chunked_fwd_bwd_inplace(twin, lab)
    torch.cuda.synchronize()
    assert l1.data_ptr() == loss.data_ptr()
    assert l1.item() == l2.item() and torch.equal(logits, twin)
    # more rows than the static scratch holds: refused before any device work
    lib = lce.load_library()
    big = lce.LCE_NOALLOC_MAX_ROWS + 1
    rc = lib.ce_chunked_fwd_bwd_inplace_noalloc(0x10000000, big, 8, 8, 0x20000000, -100, 16, -1,
                                                None, 0x30000000, None, None, None)
    assert rc == 10 and "LCE_NOALLOC_MAX_ROWS" in lce.lce_status_str(rc)
