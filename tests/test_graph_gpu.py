"""The library's calls are plain kernel launches on the caller's stream (no allocation, no
memset, no synchronisation), so they can be captured into a HIP graph. Capture the CE step and
a fused linear CE call, replay each several times with eager work between the replays, and
check every replay bit for bit against the eager result."""
import pytest
import torch

import linear_cross_entropy_masked_amd as lce
from workloads import random_ce, random_flce

from _helpers import bits_to_device, gpu_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def _capture(fn, dev):
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_ce_step_graph_replays_match_eager(dev):
    inp = random_ce(300, 5003, sigma=3.0, ignore_frac=0.1, seed=51)
    pristine = bits_to_device(inp.logits, dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    logits = torch.empty_like(pristine)
    ws = torch.empty(lce.ce_chunked_workspace_size(300, 5003, 64), dtype=torch.uint8, device=dev)
    out = {}

    def step():
        torch.mul(pristine, 1, out=logits)  # a kernel, not a copy node
        loss, lse = lce.ce_chunked_fwd(logits, lab, chunk_size=64, workspace=ws)
        lce.ce_chunked_bwd_inplace(logits, lab, chunk_size=64, lse=lse, workspace=ws)
        out["loss"] = loss

    step()
    torch.cuda.synchronize()
    ref_loss, ref_grad = out["loss"].clone(), logits.clone()
    g = _capture(step, dev)
    for k in range(4):
        logits.fill_(0)  # eager work between replays, and a clobbered output
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out["loss"], ref_loss), f"replay {k}: loss"
        assert torch.equal(logits.view(torch.int16), ref_grad.view(torch.int16)), f"replay {k}"


def test_single_pass_ce_graph_replays_match_eager(dev):
    inp = random_ce(200, 40000, sigma=2.0, ignore_frac=0.2, seed=52)
    pristine = bits_to_device(inp.logits, dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    logits = torch.empty_like(pristine)
    gout = torch.tensor(1.5, dtype=torch.float32, device=dev)
    out = {}

    def step():
        torch.mul(pristine, 1, out=logits)  # a kernel, not a copy node
        out["loss"], _ = lce.ce_chunked_fwd_bwd_inplace(logits, lab, grad_output=gout)

    step()
    torch.cuda.synchronize()
    ref_loss, ref_grad = out["loss"].clone(), logits.clone()
    g = _capture(step, dev)
    for k in range(4):
        logits.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out["loss"], ref_loss), f"replay {k}: loss"
        assert torch.equal(logits.view(torch.int16), ref_grad.view(torch.int16)), f"replay {k}"


@pytest.mark.parametrize("n,h,chunk,recompute,bias_grad,transposed", [
    (333, 128, 100, False, True, False), (333, 128, 100, True, True, False),
    (333, 128, 100, True, False, False), (600, 320, 128, False, True, True)])
def test_flce_graph_replays_match_eager(dev, n, h, chunk, recompute, bias_grad, transposed):
    """Both schedules with two chunks per slice (stored logits; recomputing without grad_bias),
    the recomputing schedule one chunk at a time (with grad_bias), and every row's
    probabilities kept transposed in grad_weight's bytes and the slice."""
    v = 3001
    inp = random_flce(n, h, v, bias=True, seed=53)
    hid = bits_to_device(inp.hidden, dev)
    w = bits_to_device(inp.weight, dev)
    b = torch.from_numpy(inp.bias).to(dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    gh = torch.empty((n, h), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((v, h), dtype=torch.float32, device=dev)
    gb = torch.empty(v, dtype=torch.float32, device=dev) if bias_grad else False
    flags = lce.FLCE_RECOMPUTE if recompute else 0
    ws = torch.empty(lce.flce_workspace_size(n, h, v, chunk, flags), dtype=torch.uint8,
                     device=dev)
    out = {}

    def step():
        out["loss"], _, _, _, _ = lce.flce_fwd_bwd(hid, w, lab, b, chunk_size=chunk,
                                                   recompute=recompute, grad_hidden=gh,
                                                   grad_weight=gw, grad_bias=gb, workspace=ws)

    torch.cuda.synchronize()
    lce.lce_timing_read()
    lce.lce_timing_enable(True)
    try:
        step()
        torch.cuda.synchronize()
        names = {name for name, _, _ in lce.lce_timing_read()}
    finally:
        lce.lce_timing_enable(False)
    assert ("flce_probs_transposed" in names) == transposed, names
    step()
    torch.cuda.synchronize()
    outs = [gh, gw] + ([gb] if bias_grad else [])
    ref = [out["loss"].clone()] + [t.clone() for t in outs]
    g = _capture(step, dev)
    for k in range(4):
        for t in outs:
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out["loss"], ref[0]), f"replay {k}: loss"
        assert torch.equal(gh.view(torch.int16), ref[1].view(torch.int16)), f"replay {k}: gh"
        assert torch.equal(gw, ref[2]), f"replay {k}: gw"
        if bias_grad:
            assert torch.equal(gb, ref[3]), f"replay {k}: gb"
