"""Out-of-bounds write detection: every buffer a call receives sits between sentinel-filled
guard bands, and after the call the bands must be intact, the inputs unchanged byte for byte,
and (for the CE layer's strided rows) the columns v .. ld − 1 of every row untouched.

The fused linear CE keeps its bookkeeping in the workspace slice's free halves and in
grad_hidden rows it has not written yet, and may keep its probabilities in grad_weight's bytes
before writing grad_weight; these tests run every schedule, both workspace
layouts (the compact one whose workspace is the slice alone, and the extended one), paired and
unpaired chunks, and the split calls, and check that nothing lands outside the buffers. The
outputs are also checked against the oracle where the case is a parity case.
"""
import numpy as np
import pytest
import torch

import linear_cross_entropy_masked_amd as lce
import oracle
from workloads import random_ce, random_flce

from _helpers import (assert_close_rel, assert_faithful_bf16, device_to_f64, gpu_device,
                      normwise_rel)

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


class Guarded:
    """A tensor view placed `band` bytes into a larger allocation whose bytes outside the view
    hold SENTINEL (or, for inputs, whose whole content is remembered)."""

    def __init__(self, dev, shape, dtype, band=1 << 20, init=None):
        self.dtype, self.shape = dtype, tuple(shape)
        self.nbytes = int(np.prod(shape, dtype=np.int64)) * torch.empty((), dtype=dtype).element_size()
        self.band = band
        self.raw = torch.full((band + self.nbytes + band,), SENTINEL, dtype=torch.uint8, device=dev)
        self.t = self.raw[band:band + self.nbytes].view(dtype).view(self.shape)
        if init is not None:
            self.t.copy_(init)
        self.before = self.raw.clone()

    def bands_intact(self):
        lo = self.raw[:self.band]
        hi = self.raw[self.band + self.nbytes:]
        return bool((lo == SENTINEL).all().item()) and bool((hi == SENTINEL).all().item())

    def unchanged(self):
        return torch.equal(self.raw, self.before)


def bits(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)


def assert_clean(named):
    bad = [k for k, g in named.items() if g is not None and not g.bands_intact()]
    assert not bad, f"guard bands overwritten next to: {bad}"


# ------------------------------------------------------------------------------- CE layer

@pytest.mark.parametrize("n,v,ld_extra", [(37, 1000, 24), (16, 32777, 7), (5, 128256, 64),
                                          (64, 1000, 0), (600, 1000, 8), (300, 32776, 0)])
def test_ce_calls_stay_inside_their_buffers(dev, n, v, ld_extra):
    inp = random_ce(n, v, sigma=3.0, ignore_frac=0.2, seed=n + v)
    ld = v + ld_extra
    pad = torch.full((n, ld), -7.25, dtype=torch.bfloat16, device=dev)
    pad[:, :v] = bits(inp.logits, dev)
    ws_bytes = lce.ce_chunked_workspace_size(n, v, 16)
    ref = oracle.ce_masked_sum(oracle.bf16_bits_to_f64(inp.logits), inp.labels)

    def fresh():
        g = {
            "logits": Guarded(dev, (n, ld), torch.bfloat16, init=pad),
            "labels": Guarded(dev, (n,), torch.int32,
                              init=torch.from_numpy(inp.labels).to(dev)),
            "loss": Guarded(dev, (), torch.float32),
            "lse": Guarded(dev, (n,), torch.float32),
            "status": Guarded(dev, (), torch.int32),
            "ws": Guarded(dev, (ws_bytes,), torch.uint8, band=4 << 20),
        }
        return g

    def logits_view(g):
        return g["logits"].t[:, :v]

    def padding_untouched(g):
        return torch.equal(g["logits"].t[:, v:], pad[:, v:])

    # forward, then the out-of-place backward into a strided gradient, then in place
    g = fresh()
    loss, lse = lce.ce_chunked_fwd(logits_view(g), g["labels"].t, chunk_size=16,
                                   status=g["status"].t, workspace=g["ws"].t)
    grad = Guarded(dev, (n, ld), torch.bfloat16, init=torch.full((n, ld), 3.5,
                                                                 dtype=torch.bfloat16))
    lce.ce_chunked_bwd(logits_view(g), g["labels"].t, out=grad.t[:, :v], lse=lse,
                       workspace=g["ws"].t)
    torch.cuda.synchronize()
    assert_clean(dict(g, grad=grad))
    assert g["logits"].unchanged() and g["labels"].unchanged()
    assert bool((grad.t[:, v:] == 3.5).all().item()), "gradient padding columns written"
    assert_close_rel(float(loss.item()), ref.loss, 1e-5)
    assert_faithful_bf16(device_to_f64(grad.t[:, :v]), ref.grad)

    g = fresh()
    lce.ce_chunked_bwd_inplace(logits_view(g), g["labels"].t, lse=None, status=g["status"].t,
                               workspace=g["ws"].t)
    torch.cuda.synchronize()
    assert_clean(g)
    assert g["labels"].unchanged() and padding_untouched(g)
    assert_faithful_bf16(device_to_f64(logits_view(g)), ref.grad)

    g = fresh()
    loss2, lse2 = lce.ce_chunked_fwd_bwd_inplace(logits_view(g), g["labels"].t,
                                                 return_lse=True, status=g["status"].t,
                                                 workspace=g["ws"].t)
    torch.cuda.synchronize()
    assert_clean(g)
    assert g["labels"].unchanged() and padding_untouched(g)
    assert float(loss2.item()) == float(loss.item())
    assert_faithful_bf16(device_to_f64(logits_view(g)), ref.grad)

    g = fresh()
    rows = Guarded(dev, (n,), torch.float32)
    lse3 = Guarded(dev, (n,), torch.float32)
    lab = g["labels"].t
    lib = lce.load_library()
    rc = lib.ce_rows_fwd(logits_view(g).data_ptr(), n, v, ld, lab.data_ptr(), -100, 16,
                         rows.t.data_ptr(), lse3.t.data_ptr(), g["status"].t.data_ptr(),
                         g["ws"].t.data_ptr(), ws_bytes,
                         torch.cuda.current_stream(dev).cuda_stream)
    assert rc == 0
    up = Guarded(dev, (n,), torch.float32, init=torch.linspace(0.5, 2.0, n))
    lce.ce_rows_bwd(logits_view(g), lab, up.t, inplace=True, lse=lse3.t, workspace=g["ws"].t)
    torch.cuda.synchronize()
    assert_clean(dict(g, rows=rows, lse3=lse3, up=up))
    assert padding_untouched(g) and g["labels"].unchanged() and up.unchanged()


# -------------------------------------------------------------------------- fused layer

FLCE_CASES = [
    # n, h, v, chunk, bias, grad_bias, recompute, accumulate: every row's probabilities kept
    # transposed in grad_weight's bytes and the slice (two segments; four grad_weight ranges
    # and padding tokens; grad_hidden split partials below them; all of Pᵀ in the slice),
    # paired 16-bit logits (a batch too long for that, even and odd chunk counts), paired
    # recompute, unpaired recompute with grad_bias, the extended layout (h not a multiple of
    # 64; chunks under 64 rows), V not a multiple of 64
    (200, 128, 1500, 64, True, True, False, False),
    (600, 320, 3001, 128, False, False, False, False),
    (300, 256, 9000, 64, False, False, False, False),
    (64, 64, 300, 64, True, True, False, False),
    (512, 128, 3000, 128, True, True, False, False),
    (192, 128, 1500, 64, False, False, True, False),
    (300, 128, 2001, 100, True, True, True, True),
    (130, 40, 1000, 32, True, True, False, False),
    (257, 64, 513, 40, False, False, True, False),
    (96, 192, 32777, 64, True, True, False, True),
]


def flce_guarded(dev, inp, chunk, bias_grad, recompute, accumulate, lse_out=True):
    n, h = inp.hidden.shape
    v = inp.weight.shape[0]
    flags = (lce.FLCE_RECOMPUTE if recompute else 0) | (lce.FLCE_ACCUMULATE if accumulate else 0)
    rng = np.random.default_rng(n + v)
    g = {
        "hidden": Guarded(dev, (n, h), torch.bfloat16, init=bits(inp.hidden, dev)),
        "weight": Guarded(dev, (v, h), torch.bfloat16, init=bits(inp.weight, dev)),
        "labels": Guarded(dev, (n,), torch.int32, init=torch.from_numpy(inp.labels).to(dev)),
        "bias": None if inp.bias is None else Guarded(dev, (v,), torch.float32,
                                                      init=torch.from_numpy(inp.bias)),
        "loss": Guarded(dev, (), torch.float32),
        "lse": Guarded(dev, (n,), torch.float32) if lse_out else None,
        "gh": Guarded(dev, (n, h), torch.bfloat16, band=4 << 20),
        "gw": Guarded(dev, (v, h), torch.float32, band=4 << 20,
                      init=torch.from_numpy(rng.normal(0, 0.01, (v, h)).astype(np.float32))
                      if accumulate else None),
        "gb": None,
        "status": Guarded(dev, (), torch.int32),
        "ws": Guarded(dev, (lce.flce_workspace_size(n, h, v, chunk, flags),), torch.uint8,
                      band=4 << 20),
    }
    if bias_grad:
        g["gb"] = Guarded(dev, (v,), torch.float32,
                          init=torch.from_numpy(rng.normal(0, 0.01, v).astype(np.float32))
                          if accumulate else None)
    init = None
    if accumulate:
        init = (g["gw"].t.double().cpu().numpy(),
                None if g["gb"] is None else g["gb"].t.double().cpu().numpy())
    return g, init


@pytest.mark.parametrize("n,h,v,chunk,bias,grad_bias,recompute,accumulate", FLCE_CASES)
def test_flce_stays_inside_its_buffers(dev, n, h, v, chunk, bias, grad_bias, recompute,
                                       accumulate):
    inp = random_flce(n, h, v, weight_sigma=0.2, bias=bias, ignore_frac=0.1, seed=3 * n + v)
    g, init = flce_guarded(dev, inp, chunk, grad_bias, recompute, accumulate)
    t = lambda k: None if g[k] is None else g[k].t  # noqa: E731
    loss, gh, gw, gb, _ = lce.flce_fwd_bwd(
        t("hidden"), t("weight"), t("labels"), t("bias"), chunk_size=chunk, recompute=recompute,
        accumulate=accumulate, grad_hidden=t("gh"), grad_weight=t("gw"),
        grad_bias=t("gb") if grad_bias else False, status=t("status"), workspace=t("ws"))
    torch.cuda.synchronize()
    assert_clean(g)
    for k in ("hidden", "weight", "labels", "bias"):
        assert g[k] is None or g[k].unchanged(), f"input {k} was written"
    ref = oracle.flce(inp.hidden, inp.weight, inp.labels, bias=inp.bias,
                      grad_weight_init=None if init is None else init[0])
    assert_close_rel(float(loss.item()), ref.loss, 1e-5)
    assert normwise_rel(device_to_f64(gh), ref.grad_hidden) <= 1e-2
    assert normwise_rel(device_to_f64(gw), ref.grad_weight) <= 1e-3
    if grad_bias:
        db = ref.grad_bias + (0.0 if init is None or init[1] is None else init[1])
        assert normwise_rel(device_to_f64(gb), db) <= 1e-4


@pytest.mark.parametrize("n,h,v,chunk,bias", [(192, 128, 1500, 64, True), (130, 40, 1000, 32, False),
                                              (300, 128, 2001, 100, True)])
def test_flce_split_calls_stay_inside_their_buffers(dev, n, h, v, chunk, bias):
    inp = random_flce(n, h, v, weight_sigma=0.2, bias=bias, ignore_frac=0.1, seed=5 * n + v)
    g, _ = flce_guarded(dev, inp, chunk, bias, False, False)
    t = lambda k: None if g[k] is None else g[k].t  # noqa: E731
    lib = lce.load_library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    ws_bytes = g["ws"].nbytes
    ptr = lambda k: None if g[k] is None else g[k].t.data_ptr()  # noqa: E731
    rc = lib.flce_fwd(ptr("hidden"), ptr("weight"), ptr("bias"), ptr("labels"), n, h, v, -100,
                      chunk, -1, ptr("loss"), ptr("lse"), ptr("status"), ptr("ws"), ws_bytes,
                      stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert_clean(g)
    g["lse"].before = g["lse"].raw.clone()  # the forward's output is the backward's input
    rc = lib.flce_bwd(ptr("hidden"), ptr("weight"), ptr("bias"), ptr("labels"), ptr("lse"), n, h,
                      v, -100, chunk, -1, 0, None, ptr("gh"), ptr("gw"), ptr("gb"), ptr("status"),
                      ptr("ws"), ws_bytes, stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert_clean(g)
    for k in ("hidden", "weight", "labels", "bias", "lse"):
        assert g[k] is None or g[k].unchanged(), f"{k} was written by the backward"
    ref = oracle.flce(inp.hidden, inp.weight, inp.labels, bias=inp.bias)
    assert_close_rel(float(t("loss").item()), ref.loss, 1e-5)
    assert normwise_rel(device_to_f64(t("gh")), ref.grad_hidden) <= 1e-2
    assert normwise_rel(device_to_f64(t("gw")), ref.grad_weight) <= 1e-3
