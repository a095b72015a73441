"""Extended correctness sweep on the GPU: the random-case generators of
test_random_sweep_gpu.py drawn from further seeds, each case checked against the oracle with the
same bars, plus paired chunks of 2048 rows (grad_weight over K = 4096 on 256 x 256 tiles).

Not collected by pytest (the default suite keeps its fixed cases); run it by hand:

    python tests/sweep_extended.py [--seeds S] [--per-kind K]

Every case is printed before it runs. A transposed-schedule case whose shape the transposed plan
cannot take (it then runs paired, still checked against the oracle) is reported as a note; any
other assertion is a failure, and the exit status is 1 when there is one.
"""
import argparse
import os
import sys
import time
import traceback

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import test_random_sweep_gpu as sweep  # noqa: E402


def wide_pair_cases(k, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(k):
        h = 64 * int(rng.integers(1, 3))
        n = int(rng.integers(4096, 7000))
        v = int(rng.integers(300, 2000))
        bias = bool(rng.random() < 0.5)
        out.append(dict(
            n=n, h=h, v=v, chunk=2048, bias=bias, bias_grad=bias and bool(rng.random() < 0.5),
            recompute=bool(rng.random() < 0.5), ignore=float(rng.uniform(0, 0.4)),
            count=None if rng.random() < 0.6 else int(rng.integers(1, 2 * n + 2)),
            g=None if rng.random() < 0.6 else float(rng.normal(0, 2)),
            wsig=float(rng.uniform(0.01, 0.2)), seed=int(rng.integers(1 << 30))))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--seeds", type=int, default=5, help="seeds per generator")
    ap.add_argument("--per-kind", type=int, default=30, help="cases per generator and seed")
    ap.add_argument("--first-seed", type=int, default=8000)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    s0, k = args.first_seed, args.per_kind
    cases = []
    for s in range(args.seeds):
        cases += [("ce", c) for c in sweep._ce_cases(k=k, seed=s0 + s)]
        cases += [("flce", c) for c in sweep._flce_cases(k=k, seed=s0 + 100 + s)]
        cases += [("paired", c) for c in sweep._flce_paired_cases(k=k, seed=s0 + 200 + s)]
        cases += [("transposed", c) for c in sweep._flce_transposed_cases(k=k, seed=s0 + 300 + s)]
    cases += [("paired_wide", c) for c in wide_pair_cases(k, s0 + 400)]
    print(f"{len(cases)} cases", flush=True)
    fails, notes = [], 0
    t0 = time.time()
    keys = ("n", "h", "v", "chunk", "recompute", "bias", "bias_grad", "ld_extra")
    for i, (kind, c) in enumerate(cases):
        name = f"{i} {kind} " + " ".join(f"{key}={c[key]}" for key in keys if key in c)
        print("case", name, flush=True)
        try:
            if kind == "ce":
                sweep.test_ce_random_case(dev, c)
            elif kind == "transposed":
                sweep.test_flce_random_transposed_case(dev, c)
            else:
                sweep._check_flce_case(dev, c)
        except AssertionError as e:
            msg = str(e)
            if kind == "transposed" and "flce_to_probs" in msg and "flce_probs_transposed" not in msg:
                notes += 1
                print("  note: the transposed plan cannot take this shape (the paired schedule "
                      "ran and matched the oracle)", flush=True)
                continue
            fails.append(name)
            print("  FAILED:", "".join(traceback.format_exception_only(type(e), e))[:400],
                  flush=True)
    print(f"done in {time.time() - t0:.0f} s: {len(cases) - len(fails)} of {len(cases)} match "
          f"the oracle ({notes} transposed-generator shapes ran paired)", flush=True)
    for f in fails:
        print("failed:", f, flush=True)
    return 1 if fails else 0


if __name__ == "__main__":
    sys.exit(main())
