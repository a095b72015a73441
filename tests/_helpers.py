"""Shared test utilities: device transfer of generator bits, bf16 ulp, tolerance checks."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch


def gpu_device():
    """cuda:0 with the HIP library loaded; skips only when there is no GPU at all."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_masked_amd as lce
    lce.load_library()  # a missing library is a failure on a GPU machine, not a skip
    return torch.device("cuda:0")


def bits_to_device(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def device_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits; subnormal spacing 2^-133)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def assert_faithful_bf16(got: np.ndarray, exact: np.ndarray, what: str = "grad"):
    """Every element within one bf16 ulp of the exact value (faithful rounding)."""
    diff = np.abs(got - exact)
    ulp = bf16_ulp(exact)
    bad = diff > ulp
    if bad.any():
        idx = np.argwhere(bad)[:5]
        msg = ", ".join(f"{tuple(i)}: got {got[tuple(i)]!r} exact {exact[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} elements off by more than 1 bf16 ulp: {msg}")


def assert_close_rel(got: float, exact: float, rel: float, what: str = "loss"):
    if exact == 0.0:
        assert got == 0.0, f"{what}: expected exactly 0, got {got}"
        return
    err = abs(got - exact) / abs(exact)
    assert err <= rel, f"{what}: rel err {err:.3e} > {rel:.1e} (got {got!r}, exact {exact!r})"


def normwise_rel(got: np.ndarray, exact: np.ndarray) -> float:
    den = np.linalg.norm(exact)
    num = np.linalg.norm(got - exact)
    return float(num / den) if den > 0 else float(num)


def host_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def oracle_ce_rows_parallel(bits: np.ndarray, labels: np.ndarray, count: int, rows_per_task=512):
    """Oracle per-row loss terms and lse for every row, computed block-parallel on the host.

    Rows are independent in the oracle's definition, so splitting them across threads changes
    no value; the loss is s · Σ row_loss.
    """
    import oracle
    n = bits.shape[0]
    row_loss = np.zeros(n)
    lse = np.zeros(n)

    def task(r0):
        r1 = min(n, r0 + rows_per_task)
        r = oracle.ce_masked_sum_bits(bits[r0:r1], labels[r0:r1], num_label_tokens=count,
                                      grad_rows=np.empty(0, np.int64), row_block=128)
        row_loss[r0:r1] = r.row_loss
        lse[r0:r1] = r.lse

    with ThreadPoolExecutor(host_threads()) as ex:
        list(ex.map(task, range(0, n, rows_per_task)))
    return row_loss, lse
