#!/usr/bin/env python3
"""Benchmark of the masked cross-entropy hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one forward+backward pass of each layer of the hot path over one batch of seeded
synthetic input already resident in HBM:
  * fused linear CE on the Llama3-8B-shaped head: hidden [8192, 4096] bf16, weight
    [128256, 4096] bf16, no bias, 5% ignored labels, chunk 1024 (loss, grad_hidden, fp32
    grad_weight) — this is `value` (tokens/s), with the bf16 MFMA roofline;
  * chunked masked CE on [16384, 128256] bf16 logits (spiked labels, 5% ignored, chunk 1024,
    in-place backward) — reported under "ce_only" with its HBM roofline, as the two calls
    (forward, then in-place backward) and, under "ce_only.single_pass", as the one call that
    does both when the upstream gradient is known (each labelled row read once);
  * fused linear CE on the small model (hidden [2048, 768], weight [32777, 768], bias, chunk
    512; loss and all four gradients) — reported under "small_model" with the oracle timed on
    the whole workload beside it;
  * fused linear CE on the long-context packed workload (hidden [32768, 8192], weight
    [128256, 8192], 8 documents, chunk 2048) with the recomputing schedule — reported under
    "long_context" (at most 3 timed steps; --no-long-context skips it).

Prints one JSON line. Timing uses hipEvents recorded on the stream the library launches on;
the in-place CE backward destroys its input, so the logits are restored from a pristine copy
between steps, outside the timed events. `value` and `ms_per_step` time the K steps back to
back; each workload's "timing" also gives the median / min / mean of the steps timed one by
one, warm (back to back) and cold (the 256 MB MALL and the L2s flushed by a 512 MB write before
each step, outside the events).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "FLCE fwd+bwd tokens/s (H4096,V128256) % MFMA peak; CE-only HBM GB/s % peak"

FLCE_WORKLOAD = "flce_8192x4096x128256"
SMALL_WORKLOAD = "flce_2048x768x32777"
LONG_WORKLOAD = "flce_32768x8192x128256_packed"
CE_WORKLOAD = "ce_16384x128256"
PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_cross_entropy_masked_amd", "csrc")


def source_digest() -> str:
    """Hash of the HIP sources: stored HBM-traffic counters are only valid for this digest."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if still current."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{kernel}@{workload}")
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


# rocprofv3 kernel names -> the library's launch-timing names (first match wins)
KERNEL_NAMES = [
    ("EpiLogits", "flce_gemm_logits"), ("EpiLseOnly", "flce_gemm_logits"),
    ("EpiProbs", "flce_gemm_probs"), ("EpiGradHidden", "flce_gemm_grad_hidden"),
    ("EpiPartial", "flce_gemm_grad_hidden"), ("EpiGradWeight", "flce_gemm_grad_weight"),
    ("slice_row_lse_kernel", "flce_row_lse"), ("slice_bias_grad_kernel", "flce_bias_grad"),
    ("slice_to_probs_kernel", "flce_to_probs"), ("shifted_to_probs_kernel", "flce_to_probs"),
    ("shifted_to_probs_p_kernel", "flce_probs_transposed"),
    ("shifted_bias_grad_kernel", "flce_bias_grad"), ("onehot_weight_fix_kernel", "flce_onehot_fix"),
    ("grad_hidden_reduce_kernel", "flce_grad_hidden_reduce"), ("fill_zero", "fill_zero"),
    ("label_rank_kernel", "flce_label_sort"), ("label_prep_kernel", "label_prep"),
    ("loss_finish_kernel", "loss_reduce"), ("loss_accumulate_kernel", "flce_loss_acc"),
    ("state_move_kernel", "flce_loss_acc"), ("loss_reduce_kernel", "loss_reduce"),
    ("ce_fwd_rows_kernel", "ce_fwd_rows"), ("ce_bwd_rows_kernel", "ce_bwd_rows"),
    ("ce_fused_rows_kernel", "ce_fused_rows"),
]
CALIB_BYTES = 1 << 30  # bytes read and bytes written by one launch of the calibration copy


def copy_calibration(torch):
    """Three launches of a plain elementwise copy (negation) of 1 GiB of bf16: what FETCH_SIZE
    and WRITE_SIZE read for it converts the counters of the library's kernels to bytes."""
    dev = torch.device("cuda:0")
    src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _counter_means(run_dir, counter):
    """Mean of `counter` per dispatch, per kernel name, over every counter_collection.csv."""
    import csv
    import glob
    tot, disp = {}, {}
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                k = r["Kernel_Name"]
                tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
                disp.setdefault(k, set()).add(r["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


def record_traffic(workload, fetch_dir, write_dir):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) of
    `bench.py --only <layer> --copy-calibration` into HBM bytes per launch of each library
    kernel, scaled by the calibration copy's readings, and store them in profiles/traffic.json
    under the current source digest."""
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")

    def calib(m):
        ks = [k for k in m if "neg_kernel" in k]
        if not ks:
            raise SystemExit("calibration copy kernel not found in the counter run")
        return CALIB_BYTES / (max(m[k] for k in ks) * 1024.0)

    f_scale, w_scale = calib(fetch), calib(write)
    out = {}
    for m, scale, key in ((fetch, f_scale, "read_bytes"), (write, w_scale, "write_bytes")):
        for k, kib in m.items():
            name = next((n for sub, n in KERNEL_NAMES if sub in k), None)
            if name is None:
                continue
            rec = out.setdefault(name, {"raw_kib": {}})
            rec[key] = rec.get(key, 0.0) + kib * 1024.0 * scale
            rec["raw_kib"][key] = rec["raw_kib"].get(key, 0.0) + kib
    path = os.path.join(PROFILE_DIR, "traffic.json")
    table = {}
    if os.path.exists(path):
        with open(path) as f:
            table = json.load(f)
    digest = source_digest()
    # a recording replaces the workload's earlier one (kernels a schedule no longer runs go)
    table = {k: v for k, v in table.items() if not k.endswith("@" + workload)}
    for name, rec in out.items():
        rd, wr = rec.get("read_bytes", 0.0), rec.get("write_bytes", 0.0)
        table[f"{name}@{workload}"] = {
            "bytes_per_launch": int(round(rd + wr)), "read_bytes": int(round(rd)),
            "write_bytes": int(round(wr)), "raw_kib_per_dispatch": rec["raw_kib"],
            "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
            "source_digest": digest}
    os.makedirs(PROFILE_DIR, exist_ok=True)
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print(json.dumps({k: v for k, v in table.items() if k.endswith("@" + workload)}, indent=1))


N_XCD = 8  # GRBM_GUI_ACTIVE is summed over the XCDs: per-XCD active cycles = value / 8
N_SIMD = 1024  # 256 CUs x 4 SIMDs


def stored_mfma(kernel: str, workload: str):
    """MFMA counters of a kernel from the committed rocprofv3 summary, if still current."""
    path = os.path.join(PROFILE_DIR, "mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel}@{workload}")
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return {k: rec[k] for k in ("flops_per_launch", "mfma_busy_frac", "clock_ghz")}


def record_mfma(workload, pmc_dir, trace_dir):
    """Turn one rocprofv3 --pmc run (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES,
    GRBM_GUI_ACTIVE) and one --kernel-trace run of `bench.py --only <layer>` into, per MFMA
    kernel: executed bf16 flops per launch (MOPS x 512), the fraction of SIMD cycles its MFMA
    pipes were busy, and the clock the active cycles imply over the traced duration."""
    import csv
    import glob
    sums, disp = {}, {}
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                k = r["Kernel_Name"]
                d = sums.setdefault(k, {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                disp.setdefault(k, set()).add(r["Dispatch_Id"])
    durs = {}
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                durs.setdefault(r["Kernel_Name"], []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    path = os.path.join(PROFILE_DIR, "mfma.json")
    table = {}
    if os.path.exists(path):
        with open(path) as f:
            table = json.load(f)
    digest = source_digest()
    table = {k: v for k, v in table.items() if not k.endswith("@" + workload)}
    for k, d in sums.items():
        mops = d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        name = next((n for sub, n in KERNEL_NAMES if sub in k), None)
        if name is None or mops <= 0 or k not in durs:
            continue
        n = len(disp[k])
        active = d["GRBM_GUI_ACTIVE"] / n / N_XCD
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / n
        t = sorted(durs[k])[len(durs[k]) // 2]
        table[f"{name}@{workload}"] = {
            "flops_per_launch": mops / n * 512, "mfma_busy_frac": round(busy / (active * N_SIMD), 4),
            "clock_ghz": round(active / t / 1e9, 3), "median_launch_ms": round(t * 1e3, 4),
            "dispatches": n, "source_digest": digest}
    os.makedirs(PROFILE_DIR, exist_ok=True)
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print(json.dumps({k: v for k, v in table.items() if k.endswith("@" + workload)}, indent=1))


def ce_algorithmic_bytes(n, v, nvalid):
    """Bytes the method must move: forward reads each labelled row once; the in-place backward
    reads each labelled row and writes every row (ignored rows are zero-filled)."""
    fwd = nvalid * v * 2
    bwd_read = nvalid * v * 2
    bwd_write = n * v * 2
    return fwd, bwd_read + bwd_write


def timed_kernels(torch, lce, stream, step, steps):
    """Run `steps` more steps with the library's per-launch hipEvents on; returns (steps,
    instrumented ms/step, [(kernel, total ms, launches)])."""
    lce.lce_timing_enable(True)
    lce.lce_timing_read()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    kernels = lce.lce_timing_read()
    lce.lce_timing_enable(False)
    return steps, ev[0].elapsed_time(ev[1]) / steps, kernels


FLUSH_BYTES = 512 << 20  # twice the MI355X's 256 MB MALL: a write of this size evicts it


def per_step_times(torch, stream, step, steps, flush=None):
    """Each of `steps` steps timed alone with a hipEvent pair on `stream`; `flush` (run before
    each step, outside the events) makes every step start with cold caches. Returns
    {median_ms, min_ms, mean_ms, steps}."""
    evs = []
    for _ in range(steps):
        if flush is not None:
            flush()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        step()
        e[1].record(stream)
        evs.append(e)
    torch.cuda.synchronize()
    return step_stats([e[0].elapsed_time(e[1]) for e in evs])


def step_stats(times_ms):
    t = sorted(times_ms)
    med = t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])
    return {"median_ms": round(med, 4), "min_ms": round(t[0], 4),
            "mean_ms": round(sum(t) / len(t), 4), "steps": len(t)}


def make_flush(torch, dev):
    """A 512 MB device buffer rewritten by each call (a plain fill kernel)."""
    buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    counter = [0]

    def flush():
        counter[0] += 1
        buf.fill_(counter[0])
    return flush


def gemm_bytes(kernel, w, launches, stored_slice=True, transposed=False):
    """Algorithmic HBM bytes of one launch of an FLCE product (averaged over its `launches`
    per step): each operand read once, each result written once. The stored-logits schedules
    write each chunk's logits as 16-bit shifted values; the recomputing schedule stores none.
    Paired chunks: grad_hidden per chunk, grad_weight once per two chunks (K = 2C) adding
    into its fp32 accumulator (written by the first launch, read and written by the others).
    Transposed probabilities (every row's kept at once): grad_hidden is one product over all
    rows, grad_weight one product per vocabulary range over all rows (K = n), each reading
    the hidden rows and writing its range of grad_weight once."""
    c, h, v, n = w.chunk_size, w.h, w.v, w.n
    if kernel == "flce_gemm_logits":  # W and the hidden chunk in; 16-bit logits out (stored)
        return 2 * v * h + 2 * c * h + (2 * c * v if stored_slice else 0)
    if kernel == "flce_gemm_probs":  # W and the hidden chunk in; bf16 probabilities out
        return 2 * v * h + 2 * c * h + 2 * c * v
    if kernel == "flce_gemm_grad_hidden":  # probabilities and W in; grad_hidden rows out
        if transposed:
            return (2 * n * v + 2 * v * h + 2 * n * h) / launches
        return 2 * c * v + 2 * v * h + 2 * c * h
    if kernel == "flce_gemm_grad_weight":  # probabilities and hidden in; fp32 grad_weight
        if transposed:
            return (2 * n * v + 2 * n * h * launches + 4 * v * h) / launches
        k = n / launches
        acc = (4 + 8 * (launches - 1)) * v * h / launches
        return 2 * k * v + 2 * k * h + acc
    raise KeyError(kernel)


def gemm_roofline(kernel, flops, nbytes, avg_ms):
    """Roofline of one product launch: it is bound by whichever floor is higher, flops at the
    bf16 MFMA peak or algorithmic bytes at the HBM peak; the other figure is kept beside it."""
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    tflops = flops / (avg_ms * 1e-3) / 1e12
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    mfma = {"achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    hbm = {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": int(nbytes)}
    if t_hbm > t_mfma:
        roof = {"bound": "hbm", "kernel": kernel, **hbm, "mfma": mfma}
    else:
        roof = {"bound": "mfma", "kernel": kernel, **mfma, "hbm": hbm}
    roof["avg_launch_ms"] = round(avg_ms, 4)
    return roof


def run_flce(args, torch, lce, workloads, name=None, recompute=False, steps=None, warmup=None):
    w = workloads.WORKLOADS[name or FLCE_WORKLOAD]
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    t0 = time.time()
    inp = workloads.make_flce_inputs(w, seed=0)
    gen_s = time.time() - t0
    dev = torch.device("cuda:0")
    import numpy as np
    hid = torch.from_numpy(inp.hidden.view(np.int16)).view(torch.bfloat16).to(dev)
    wt = torch.from_numpy(inp.weight.view(np.int16)).view(torch.bfloat16).to(dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    gh = torch.empty((w.n, w.h), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((w.v, w.h), dtype=torch.float32, device=dev)
    gb = None if bias is None else torch.empty(w.v, dtype=torch.float32, device=dev)
    flags = lce.FLCE_RECOMPUTE if recompute else 0
    ws = torch.empty(lce.flce_workspace_size(w.n, w.h, w.v, w.chunk_size, flags),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    nvalid = int((inp.labels != -100).sum())

    def step():
        return lce.flce_fwd_bwd(hid, wt, lab, bias, chunk_size=w.chunk_size, grad_hidden=gh,
                                grad_weight=gw, grad_bias=gb if gb is not None else False,
                                workspace=ws, recompute=recompute)

    for _ in range(warmup):
        step()
    # peak extra memory of one call: its peak allocation above what it leaves behind (the
    # inputs, the caller's buffers and the outputs it returns), plus the workspace
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    kept = step()
    torch.cuda.synchronize()
    peak_extra = (torch.cuda.max_memory_allocated(dev) - torch.cuda.memory_allocated(dev)
                  + ws.numel())
    del kept
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(steps):
        loss = step()[0]
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev[0].elapsed_time(ev[1]) / steps

    # the same K steps timed one by one, warm (back to back) and cold (the MALL and L2
    # flushed by a 512 MB write before each, outside the events)
    warm = per_step_times(torch, stream, step, steps)
    cold = per_step_times(torch, stream, step, steps, flush=make_flush(torch, dev))

    # per-kernel breakdown: the same K steps again with a hipEvent pair around every launch,
    # recorded by the library on the stream it launches on
    kreps, inst_ms, kernels = timed_kernels(torch, lce, stream, step, steps)

    flops = 6.0 * w.n * w.h * w.v
    chunks = -(-w.n // w.chunk_size)
    # each MFMA kernel does one 2·n·h·v product per step (the logits twice when recomputing:
    # two kernels), over however many launches the schedule splits it into; per launch the
    # algorithmic flops and bytes are averaged over those launches
    gemm_names = ("flce_gemm_logits", "flce_gemm_probs", "flce_gemm_grad_hidden",
                  "flce_gemm_grad_weight")
    transposed = any(k[0] == "flce_probs_transposed" for k in kernels)
    gemms = [k for k in kernels if k[0] in gemm_names]
    dom = max(gemms, key=lambda k: k[1]) if gemms else None
    roof = None
    if dom:
        avg_ms = dom[1] / dom[2]
        launches = dom[2] // kreps
        roof = gemm_roofline(dom[0], 2.0 * w.n * w.h * w.v / launches,
                             gemm_bytes(dom[0], w, launches, stored_slice=not recompute,
                                        transposed=transposed), avg_ms)
        roof["traffic"] = stored_traffic(dom[0], w.name)
        roof["mfma_counters"] = stored_mfma(dom[0], w.name)
    executed = (8.0 if recompute else 6.0) * w.n * w.h * w.v
    return {
        "workload": w, "ms": ms, "wall_s": wall, "tokens_per_s": w.n / (ms * 1e-3),
        "tflops": flops / (ms * 1e-3) / 1e12, "loss": float(loss.item()), "roofline": roof,
        "executed_tflops": executed / (ms * 1e-3) / 1e12,
        "instrumented_ms": inst_ms,
        "kernels": {k[0]: {"ms_per_step": round(k[1] / kreps, 4), "launches_per_step": k[2] // kreps}
                    for k in kernels},
        "peak_extra_bytes": int(peak_extra), "slice_budget_bytes": int(w.chunk_size * w.v * 4),
        "nvalid": nvalid, "gen_s": gen_s, "chunks": chunks, "inputs": inp,
        "timing": {"back_to_back_mean_ms": round(ms, 4), "warm": warm, "cold": cold},
    }


def run_ce(args, torch, lce, workloads):
    import numpy as np
    w = workloads.WORKLOADS[CE_WORKLOAD]
    t0 = time.time()
    inp = workloads.make_ce_inputs(w, seed=0)
    gen_s = time.time() - t0
    dev = torch.device("cuda:0")
    pristine = torch.from_numpy(inp.logits.view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.empty_like(pristine)
    lab = torch.from_numpy(inp.labels).to(dev)
    ws = torch.empty(lce.ce_chunked_workspace_size(w.n, w.v, w.chunk_size), dtype=torch.uint8,
                     device=dev)
    lse = torch.empty(w.n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    nvalid = int((inp.labels != -100).sum())
    fwd_bytes, bwd_bytes = ce_algorithmic_bytes(w.n, w.v, nvalid)

    flush = make_flush(torch, dev)

    def step(timed, cold=False):
        logits.copy_(pristine)
        if cold:  # the copy's tail would otherwise sit in the MALL
            flush()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timed else None
        if timed:
            e[0].record(stream)
        loss, l = lce.ce_chunked_fwd(logits, lab, chunk_size=w.chunk_size, workspace=ws)
        if timed:
            e[1].record(stream)
        lce.ce_chunked_bwd_inplace(logits, lab, chunk_size=w.chunk_size, lse=l, workspace=ws)
        if timed:
            e[2].record(stream)
        return loss, e

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    evs = []
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        loss, e = step(True)
        evs.append(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms = fwd_ms + bwd_ms
    timing = {"warm": step_stats([e[0].elapsed_time(e[2]) for e in evs])}
    cold = [step(True, cold=True)[1] for _ in range(args.steps)]
    torch.cuda.synchronize()
    timing["cold"] = step_stats([e[0].elapsed_time(e[2]) for e in cold])
    timing["cold_fwd"] = step_stats([e[0].elapsed_time(e[1]) for e in cold])
    timing["cold_bwd"] = step_stats([e[1].elapsed_time(e[2]) for e in cold])

    kreps, inst_ms, kernels = timed_kernels(torch, lce, stream, lambda: step(False), args.steps)
    kd = {k[0]: k for k in kernels}
    roof = None
    if "ce_bwd_rows" in kd:
        k = kd["ce_bwd_rows"]
        avg_ms = k[1] / k[2]
        achieved = bwd_bytes / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "ce_bwd_rows", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "avg_launch_ms": round(avg_ms, 4),
                "traffic": stored_traffic("ce_bwd_rows", CE_WORKLOAD)}
    fwd_gbs = fwd_bytes / (fwd_ms * 1e-3) / 1e9
    tot_gbs = (fwd_bytes + bwd_bytes) / (ms * 1e-3) / 1e9
    single = run_ce_single_pass(args, torch, lce, w, pristine, logits, lab, ws, stream,
                                bwd_bytes, flush)
    return {
        "workload": w, "ms": ms, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "wall_s": wall,
        "tokens_per_s": w.n / (ms * 1e-3), "gbs": tot_gbs, "fwd_gbs": fwd_gbs,
        "bwd_gbs": bwd_bytes / (bwd_ms * 1e-3) / 1e9, "loss": float(loss.item()),
        "roofline": roof, "algorithmic_bytes": fwd_bytes + bwd_bytes, "gen_s": gen_s,
        "instrumented_ms": inst_ms,
        "kernels": {k[0]: {"ms_per_step": round(k[1] / kreps, 4), "launches_per_step": k[2] // kreps}
                    for k in kernels},
        "inputs": inp, "nvalid": nvalid, "single": single, "timing": timing,
    }


def run_ce_single_pass(args, torch, lce, w, pristine, logits, lab, ws, stream, nbytes, flush):
    """The same CE step as one call (ce_chunked_fwd_bwd_inplace): each labelled row read once
    and every row written once, so its algorithmic bytes are those of the backward alone."""
    def step(timed, cold=False):
        logits.copy_(pristine)
        if cold:
            flush()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)] if timed else None
        if timed:
            e[0].record(stream)
        loss, _ = lce.ce_chunked_fwd_bwd_inplace(logits, lab, chunk_size=w.chunk_size,
                                                 workspace=ws)
        if timed:
            e[1].record(stream)
        return loss, e

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    evs = [step(True)[1] for _ in range(args.steps)]
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    timing = {"warm": step_stats([e[0].elapsed_time(e[1]) for e in evs])}
    cold = [step(True, cold=True)[1] for _ in range(args.steps)]
    torch.cuda.synchronize()
    timing["cold"] = step_stats([e[0].elapsed_time(e[1]) for e in cold])
    kreps, _, kernels = timed_kernels(torch, lce, stream, lambda: step(False), args.steps)
    kd = {k[0]: k for k in kernels}
    roof = None
    if "ce_fused_rows" in kd:
        k = kd["ce_fused_rows"]
        avg_ms = k[1] / k[2]
        achieved = nbytes / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "ce_fused_rows", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "avg_launch_ms": round(avg_ms, 4),
                "traffic": stored_traffic("ce_fused_rows", CE_WORKLOAD)}
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.n / (ms * 1e-3), 1),
            "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "roofline": roof, "timing": timing,
            "kernels": {k[0]: {"ms_per_step": round(k[1] / kreps, 4),
                               "launches_per_step": k[2] // kreps} for k in kernels}}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("internal_api") in ("openblas", "mkl", "blis")]
        if info:
            return int(info[0]["num_threads"])
    except Exception:  # pragma: no cover
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline_flce(res):
    """The fp64 oracle on the first 4096 tokens of the same workload (all of the weight)."""
    import oracle
    inp = res["inputs"]
    k = 4096
    t0 = time.perf_counter()
    oracle.flce(inp.hidden[:k], inp.weight, inp.labels[:k], num_label_tokens=res["nvalid"],
                row_block=256)
    dt = time.perf_counter() - t0
    return {"value": round(k / dt, 2), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {k} of {res['workload'].n} tokens, full weight "
                      f"[{res['workload'].v}, {res['workload'].h}]: loss, grad_hidden, grad_weight in fp64"}


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline_flce_full(res):
    """The fp64 oracle on the whole workload (loss, grad_hidden, grad_weight, grad_bias)."""
    import oracle
    inp = res["inputs"]
    w = res["workload"]
    t0 = time.perf_counter()
    oracle.flce(inp.hidden, inp.weight, inp.labels, bias=inp.bias, row_block=256)
    dt = time.perf_counter() - t0
    return {"value": round(w.n / dt, 2), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"the whole workload ({w.n} tokens, weight [{w.v}, {w.h}], bias): loss "
                      f"and every gradient in fp64"}


def cpu_baseline_ce(res):
    """The fp64 oracle on all 16384 rows of the same logits, row blocks spread over the host
    cores (threads: numpy releases the interpreter lock inside its array operations; a process
    pool would have to fork a process that holds the GPU)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    inp = res["inputs"]
    n = res["workload"].n
    cores = host_cores()
    block = 128

    def task(r0):
        r1 = min(n, r0 + block)
        oracle.ce_masked_sum_bits(inp.logits[r0:r1], inp.labels[r0:r1],
                                  num_label_tokens=res["nvalid"], row_block=block)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        list(ex.map(task, range(0, n, block)))
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"all {n} rows of the [{n}, {res['workload'].v}] logits: loss terms and "
                      f"full gradient rows in fp64, {block}-row blocks on {cores} threads"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["flce", "small", "long", "ce"], default=None,
                    help="run one workload only (profiling): the Llama3-8B-shaped FLCE head, "
                         "the small-model FLCE (with bias), the long-context recompute FLCE, "
                         "or the CE-only logits")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the [32768, 8192] x [128256, 8192] recompute workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 1 GiB copy whose HBM counters calibrate the others")
    ap.add_argument("--record-traffic", nargs=3, metavar=("LAYER", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: store HBM bytes per launch from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of --only LAYER --copy-calibration")
    ap.add_argument("--record-mfma", nargs=3, metavar=("LAYER", "PMC_DIR", "TRACE_DIR"),
                    help="no GPU: store MFMA flops, busy fraction and clock per launch from a "
                         "rocprofv3 --pmc run (SQ_INSTS_VALU_MFMA_MOPS_BF16, "
                         "SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) and a --kernel-trace run")
    args = ap.parse_args(argv)
    if args.record_mfma:
        layer, pdir, tdir = args.record_mfma
        record_mfma({"flce": FLCE_WORKLOAD, "small": SMALL_WORKLOAD, "long": LONG_WORKLOAD,
                     "ce": CE_WORKLOAD}[layer], pdir, tdir)
        return 0
    if args.record_traffic:
        layer, fdir, wdir = args.record_traffic
        record_traffic({"flce": FLCE_WORKLOAD, "small": SMALL_WORKLOAD, "long": LONG_WORKLOAD,
                        "ce": CE_WORKLOAD}[layer], fdir, wdir)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        return 2

    import torch
    import linear_cross_entropy_masked_amd as lce
    import workloads
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    lce.load_library()
    if args.copy_calibration:
        copy_calibration(torch)

    out = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded PCG64 normals rounded to bf16; labels uniform with ignore holes)"}
    fl = ce = None
    if args.only in (None, "flce"):
        fl = run_flce(args, torch, lce, workloads)
        w = fl["workload"]
        print(f"# flce {w.name}: {fl['ms']:.3f} ms/step, {fl['tokens_per_s']:.0f} tokens/s, "
              f"{fl['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        out.update({
            "value": round(fl["tokens_per_s"], 1), "ms_per_step": round(fl["ms"], 4),
            "config": {"workload": w.name, "tokens": w.n, "hidden": w.h, "vocab": w.v,
                       "chunk_size": w.chunk_size, "bias": False, "ignored": w.n - fl["nvalid"],
                       "outputs": "loss, grad_hidden bf16, grad_weight fp32"},
            "tflops": round(fl["tflops"], 2),
            "mfma_frac": round(fl["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
            "roofline": fl["roofline"],
            "kernels": fl["kernels"],
            "peak_extra_bytes": fl["peak_extra_bytes"],
            "slice_budget_bytes": fl["slice_budget_bytes"],
            "loss": fl["loss"], "timing": fl["timing"],
        })
    if args.only in (None, "small"):
        sm = run_flce(args, torch, lce, workloads, name=SMALL_WORKLOAD)
        w = sm["workload"]
        print(f"# flce {w.name}: {sm['ms']:.3f} ms/step, {sm['tokens_per_s']:.0f} tokens/s",
              file=sys.stderr, flush=True)
        small = {
            "workload": w.name, "tokens": w.n, "hidden": w.h, "vocab": w.v,
            "chunk_size": w.chunk_size, "bias": True,
            "outputs": "loss, grad_hidden bf16, grad_weight fp32, grad_bias fp32",
            "ms_per_step": round(sm["ms"], 4), "tokens_per_s": round(sm["tokens_per_s"], 1),
            "tflops": round(sm["tflops"], 2),
            "mfma_frac": round(sm["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
            "roofline": sm["roofline"], "kernels": sm["kernels"], "timing": sm["timing"],
            "peak_extra_bytes": sm["peak_extra_bytes"],
            "slice_budget_bytes": sm["slice_budget_bytes"], "loss": sm["loss"]}
        if not args.no_cpu_baseline:
            small["cpu_baseline"] = cpu_baseline_flce_full(sm)
        if args.only == "small":
            out.update({"value": small["tokens_per_s"], "ms_per_step": small["ms_per_step"],
                        "config": {"workload": w.name, "tokens": w.n, "hidden": w.h,
                                   "vocab": w.v, "chunk_size": w.chunk_size, "bias": True},
                        "roofline": sm["roofline"]})
        out["small_model"] = small
        del sm
        torch.cuda.empty_cache()
    if args.only == "long" or (args.only is None and not args.no_long_context):
        lc = run_flce(args, torch, lce, workloads, name=LONG_WORKLOAD, recompute=True,
                      steps=min(args.steps, 3), warmup=1)
        w = lc["workload"]
        print(f"# flce {w.name} (recompute): {lc['ms']:.3f} ms/step, "
              f"{lc['tokens_per_s']:.0f} tokens/s", file=sys.stderr, flush=True)
        out["long_context"] = {
            "workload": w.name, "schedule": "recompute (logits GEMM twice: 8*N*H*V flop)",
            "tokens": w.n, "hidden": w.h, "vocab": w.v, "chunk_size": w.chunk_size,
            "steps": min(args.steps, 3), "ms_per_step": round(lc["ms"], 3),
            "tokens_per_s": round(lc["tokens_per_s"], 1),
            "model_tflops": round(lc["tflops"], 2), "executed_tflops": round(lc["executed_tflops"], 2),
            "mfma_frac_executed": round(lc["executed_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
            "roofline": lc["roofline"], "kernels": lc["kernels"], "timing": lc["timing"],
            "peak_extra_bytes": lc["peak_extra_bytes"], "slice_budget_bytes": lc["slice_budget_bytes"],
            "loss": lc["loss"]}
        if args.only == "long":
            out.update({"value": round(lc["tokens_per_s"], 1), "ms_per_step": round(lc["ms"], 4),
                        "config": {"workload": w.name, "tokens": w.n, "hidden": w.h,
                                   "vocab": w.v, "chunk_size": w.chunk_size,
                                   "schedule": "recompute"},
                        "roofline": lc["roofline"]})
        del lc
        torch.cuda.empty_cache()
    if args.only in (None, "ce"):
        ce = run_ce(args, torch, lce, workloads)
        w = ce["workload"]
        print(f"# ce {w.name}: {ce['ms']:.3f} ms/step, {ce['gbs']:.0f} GB/s; single pass "
              f"{ce['single']['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
        ce_obj = {
            "workload": w.name, "ms_per_step": round(ce["ms"], 4),
            "fwd_ms": round(ce["fwd_ms"], 4), "bwd_ms": round(ce["bwd_ms"], 4),
            "tokens_per_s": round(ce["tokens_per_s"], 1), "GB_per_s": round(ce["gbs"], 1),
            "hbm_frac": round(ce["gbs"] / HBM_PEAK_GBS, 4),
            "fwd_GB_per_s": round(ce["fwd_gbs"], 1), "bwd_GB_per_s": round(ce["bwd_gbs"], 1),
            "algorithmic_bytes": ce["algorithmic_bytes"], "roofline": ce["roofline"],
            "kernels": ce["kernels"], "loss": ce["loss"], "single_pass": ce["single"],
            "timing": ce["timing"],
        }
        if fl is None:
            out.update({"value": round(ce["tokens_per_s"], 1), "ms_per_step": round(ce["ms"], 4),
                        "config": {"workload": w.name, "tokens": w.n, "vocab": w.v,
                                   "chunk_size": w.chunk_size},
                        "roofline": ce["roofline"]})
        out["ce_only"] = ce_obj
    if not args.no_cpu_baseline:
        if fl is not None:
            out["cpu_baseline"] = cpu_baseline_flce(fl)
        if ce is not None:
            (out["ce_only"] if "ce_only" in out and fl is not None else out)["cpu_baseline"] = \
                cpu_baseline_ce(ce)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
