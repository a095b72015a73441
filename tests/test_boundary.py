"""CPU checks of the C-ABI library: it loads, exports every declared symbol, and rejects bad
arguments with the documented status codes before touching the GPU (no kernel is launched).

The calls pass fake device addresses. A call whose arguments are otherwise valid gets past
validation, so it is made only where no GPU is visible: there it must stop at the device check
(HIP when no device can be selected, DEVICE for a wrong one), which shows that validation accepted it. With a GPU present such a call would launch
kernels on the fake addresses, so those checks are skipped there."""
import ctypes
import glob
import os
import re

import pytest
import torch

import linear_cross_entropy_masked_amd as lce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL_ARG, BAD_SHAPE, BAD_CHUNK, WORKSPACE, HIP, DEVICE, BAD_FLAGS, ALIGN, OVERLAP = range(10)
SCRATCH_LIMIT = 10


def _declared_functions():
    names = []
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lce.library_path()):
        pytest.skip("library not built")
    return lce.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"ce_chunked_fwd", "ce_chunked_bwd_inplace", "flce_fwd_bwd"} <= set(names)
    raw = ctypes.CDLL(lce.library_path())
    for n in names:
        assert hasattr(raw, n), f"{n} declared in include/ but not exported"


def test_status_strings(lib):
    for code in range(11):
        assert lce.lce_status_str(code) != lce.lce_status_str(12345)
    assert lce.lce_status_str(0) == "ok"
    assert "unknown" in lce.lce_status_str(12345)


def _ws(n, v, c):
    out = ctypes.c_size_t()
    rc = lce.load_library().ce_chunked_workspace_size(n, v, c, ctypes.byref(out))
    return rc, out.value


def test_ce_workspace_size_is_small_and_validated(lib):
    rc, b = _ws(16384, 128256, 1024)
    assert rc == OK
    # O(n): no fp32 [chunk, V] slice is ever allocated by the CE layer
    assert b <= 256 + 16384 * 4 + 256
    assert _ws(-1, 10, 4)[0] == BAD_SHAPE
    assert _ws(10, 0, 4)[0] == BAD_SHAPE
    assert _ws(10, 10, 0)[0] == BAD_CHUNK
    assert lib.ce_chunked_workspace_size(10, 10, 4, None) == NULL_ARG


FAKE = 0x10000  # a 256-aligned non-null address; never dereferenced (validation fails first)
# distinct 256-aligned fake buffers, 256 MiB apart, for calls whose arguments must pass the
# overlap check
A1, A2, A3, A4, A5, A6, A7, A8, A9, A10, A11, A12 = (0x10000000 * (k + 1) for k in range(12))


AT_DEVICE_CHECK = (HIP, DEVICE)


def _no_gpu():
    """True where a call that passes validation cannot reach a kernel launch."""
    return torch.cuda.device_count() == 0


def _fwd(n=4, v=8, ld=8, logits=FAKE, labels=FAKE, chunk=2, loss=FAKE, ws=FAKE, wsb=1 << 20,
         lse=None):
    return lce.load_library().ce_chunked_fwd(logits, n, v, ld, labels, -100, chunk, -1, loss, lse,
                                             None, ws, wsb, None)


def test_ce_fwd_argument_errors(lib):
    assert _fwd(n=-1) == BAD_SHAPE
    assert _fwd(v=0) == BAD_SHAPE
    assert _fwd(ld=7) == BAD_SHAPE
    assert _fwd(n=1 << 40, ld=1 << 30, v=8) == BAD_SHAPE
    assert _fwd(chunk=0) == BAD_CHUNK
    assert _fwd(chunk=-3) == BAD_CHUNK
    assert _fwd(logits=None) == NULL_ARG
    assert _fwd(labels=None) == NULL_ARG
    assert _fwd(loss=None) == NULL_ARG
    assert _fwd(ws=None) == WORKSPACE
    assert _fwd(wsb=16) == WORKSPACE
    assert _fwd(logits=FAKE + 1) == ALIGN
    assert _fwd(labels=FAKE + 2) == ALIGN
    assert _fwd(lse=FAKE + 2) == ALIGN


def test_ce_bwd_argument_errors(lib):
    f = lib.ce_chunked_bwd
    assert f(FAKE, 4, 8, 8, FAKE, 7, FAKE, -100, 2, -1, None, None, None, FAKE, 1 << 20, None) == BAD_SHAPE
    assert f(FAKE, 4, 8, 8, None, 8, FAKE, -100, 2, -1, None, None, None, FAKE, 1 << 20, None) == NULL_ARG
    assert f(FAKE, 4, 8, 8, FAKE, 8, FAKE, -100, 0, -1, None, None, None, FAKE, 1 << 20, None) == BAD_CHUNK
    g = lib.ce_chunked_bwd_inplace
    assert g(None, 4, 8, 8, FAKE, -100, 2, -1, None, None, None, FAKE, 1 << 20, None) == NULL_ARG
    assert g(FAKE, 4, 8, 8, FAKE, -100, 2, -1, None, None, None, FAKE, 8, None) == WORKSPACE


def _fused(n=4, v=8, ld=8, logits=FAKE, labels=FAKE, chunk=2, gout=None, loss=FAKE, lse=None,
           ws=FAKE, wsb=1 << 20):
    return lce.load_library().ce_chunked_fwd_bwd_inplace(logits, n, v, ld, labels, -100, chunk,
                                                         -1, gout, loss, lse, None, ws, wsb,
                                                         None)


def test_ce_fused_argument_errors(lib):
    assert _fused(n=-1) == BAD_SHAPE
    assert _fused(v=0) == BAD_SHAPE
    assert _fused(ld=7) == BAD_SHAPE
    assert _fused(chunk=0) == BAD_CHUNK
    assert _fused(logits=None) == NULL_ARG
    assert _fused(labels=None) == NULL_ARG
    assert _fused(loss=None) == NULL_ARG
    if _no_gpu():  # n == 0 needs no rows: accepted, then stopped at the device check
        assert _fused(n=0, logits=None, labels=None, loss=A1, ws=A2) in AT_DEVICE_CHECK
    assert _fused(ws=None) == WORKSPACE
    assert _fused(wsb=16) == WORKSPACE
    assert _fused(logits=FAKE + 1) == ALIGN
    assert _fused(gout=FAKE + 2) == ALIGN
    assert _fused(lse=FAKE + 2) == ALIGN


def test_ce_rows_argument_errors(lib):
    f, b = lib.ce_rows_fwd, lib.ce_rows_bwd
    if _no_gpu():
        assert f(A1, 4, 8, 8, A2, -100, 2, A3, None, None, A4, 1 << 20, None) in AT_DEVICE_CHECK
    assert f(FAKE, 4, 8, 8, FAKE, -100, 2, None, None, None, FAKE, 1 << 20, None) == NULL_ARG
    assert f(FAKE, 4, 0, 8, FAKE, -100, 2, FAKE, None, None, FAKE, 1 << 20, None) == BAD_SHAPE
    assert f(FAKE, 4, 8, 8, FAKE, -100, 0, FAKE, None, None, FAKE, 1 << 20, None) == BAD_CHUNK
    assert f(FAKE, 4, 8, 8, FAKE, -100, 2, FAKE + 2, None, None, FAKE, 1 << 20, None) == ALIGN
    assert f(FAKE, 4, 8, 8, FAKE, -100, 2, FAKE, None, None, FAKE, 8, None) == WORKSPACE
    assert b(FAKE, 4, 8, 8, FAKE, 8, FAKE, -100, 2, None, None, None, FAKE, 1 << 20,
             None) == NULL_ARG  # grad_rows is required
    assert b(FAKE, 4, 8, 8, FAKE, 7, FAKE, -100, 2, FAKE, None, None, FAKE, 1 << 20,
             None) == BAD_SHAPE
    assert b(FAKE, 4, 8, 8, FAKE, 8, FAKE, -100, 2, FAKE + 2, None, None, FAKE, 1 << 20,
             None) == ALIGN
    assert b(FAKE, 4, 8, 8, FAKE, 8, FAKE, -100, 2, FAKE, None, None, FAKE, 8, None) == WORKSPACE


def _fws(n, h, v, c, flags=0):
    out = ctypes.c_size_t()
    rc = lce.load_library().flce_workspace_size(n, h, v, c, flags, ctypes.byref(out))
    return rc, out.value


def test_flce_workspace_is_one_slice(lib):
    # The fp32 working set of one chunk is chunk * V * 4 bytes. Liger-Kernel issue #941's
    # reply works the same arithmetic for 2 x 1024 rows of V = 32768 fp32 logits: 256 MiB.
    # With h a multiple of 64 and a chunk of at least 64 rows that slice is the whole
    # workspace, whatever n is and for either schedule.
    rc, b = _fws(2048, 768, 32768, 2048)
    assert rc == OK
    slice_bytes = 2 * 1024 * 32768 * 4
    assert slice_bytes == 256 * 1024 * 1024
    assert b == slice_bytes
    n = 1 << 20
    for flags in (0, lce.FLCE_RECOMPUTE):
        rc, b2 = _fws(n, 4096, 128256, 1024, flags)
        assert rc == OK and b2 == 1024 * 128256 * 4
        rc, b3 = _fws(32768, 8192, 128256, 2048, flags)
        assert rc == OK and b3 == 2048 * 128256 * 4
    # V not a multiple of 64: rows are padded to 64 columns (256-byte groups)
    rc, b4 = _fws(2048, 768, 32777, 512)
    assert rc == OK and b4 == 512 * 32832 * 4
    # Otherwise (h not a multiple of 64, or chunks under 64 rows) a few words per chunk row
    # sit beside the slice: lse, label logit, loss term and one (max, Σexp) pair per
    # 256-column tile; nothing grows with n.
    for h, c in ((4104, 1024), (4096, 32)):
        rc, b5 = _fws(n, h, 128256, c)
        s5 = c * 128256 * 4
        assert rc == OK and s5 < b5 <= s5 + c * (501 * 8 + 12) + 4 * 256


def test_flce_argument_errors(lib):
    assert _fws(10, 12, 100, 4)[0] == BAD_SHAPE       # h not a multiple of 8
    assert _fws(10, 0, 100, 4)[0] == BAD_SHAPE
    assert _fws(10, 16, 0, 4)[0] == BAD_SHAPE
    assert _fws(-1, 16, 10, 4)[0] == BAD_SHAPE
    assert _fws(10, 16, 10, 0)[0] == BAD_CHUNK
    assert _fws(10, 16, 10, 4, 8)[0] == BAD_FLAGS
    f = lib.flce_fwd_bwd
    args = dict(hidden=FAKE, weight=FAKE, bias=None, labels=FAKE, n=4, h=16, v=10, ign=-100,
                chunk=2, t=-1, flags=0, gout=None, loss=FAKE, lse=None, gh=None, gw=None, gb=None,
                status=None, ws=FAKE, wsb=1 << 22, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())

    assert call(weight=None) == NULL_ARG
    assert call(loss=None) == NULL_ARG
    assert call(gb=FAKE) == NULL_ARG                 # grad_bias without a bias
    assert call(flags=4) == BAD_FLAGS
    assert call(chunk=0) == BAD_CHUNK
    assert call(h=12) == BAD_SHAPE
    assert call(ws=None) == WORKSPACE
    assert call(wsb=64) == WORKSPACE
    assert call(hidden=FAKE + 8) == ALIGN
    assert call(gw=FAKE + 4) == ALIGN


def test_flce_split_argument_errors(lib):
    fwd = lib.flce_fwd
    fa = dict(hidden=FAKE, weight=FAKE, bias=None, labels=FAKE, n=4, h=16, v=10, ign=-100,
              chunk=2, t=-1, loss=FAKE, lse=FAKE, status=None, ws=FAKE, wsb=1 << 22, stream=None)

    def cf(**kw):
        return fwd(*dict(fa, **kw).values())

    assert cf(lse=None) == NULL_ARG                  # the backward needs it
    assert cf(loss=None) == NULL_ARG
    if _no_gpu():
        assert cf(n=0, hidden=None, labels=None, lse=None, weight=A1, loss=A2,
                  ws=A3) in AT_DEVICE_CHECK
    assert cf(h=12) == BAD_SHAPE
    assert cf(chunk=0) == BAD_CHUNK
    assert cf(wsb=64) == WORKSPACE
    assert cf(lse=FAKE + 2) == ALIGN
    bwd = lib.flce_bwd
    ba = dict(hidden=FAKE, weight=FAKE, bias=None, labels=FAKE, lse=FAKE, n=4, h=16, v=10,
              ign=-100, chunk=2, t=-1, flags=0, gout=None, gh=None, gw=None, gb=None, status=None,
              ws=FAKE, wsb=1 << 22, stream=None)

    def cb(**kw):
        return bwd(*dict(ba, **kw).values())

    assert cb(lse=None) == NULL_ARG
    assert cb(gb=FAKE) == NULL_ARG                   # grad_bias without a bias
    assert cb(flags=lce.FLCE_RECOMPUTE) == BAD_FLAGS  # implied, not a choice here
    assert cb(flags=8) == BAD_FLAGS
    assert cb(h=12) == BAD_SHAPE
    assert cb(ws=None) == WORKSPACE
    assert cb(gw=FAKE + 4) == ALIGN


# ---- aliasing: every buffer a call writes must be disjoint from the call's other buffers ----

def test_ce_overlapping_buffers_are_refused(lib):
    n, v = 4, 8
    fwd = lib.ce_chunked_fwd
    # workspace inside the logits, the loss inside the labels, lse over the workspace
    assert fwd(A1, n, v, v, A2, -100, 2, -1, A3, None, None, A1, 1 << 20, None) == OVERLAP
    assert fwd(A1, n, v, v, A2, -100, 2, -1, A2 + 4, None, None, A4, 1 << 20, None) == OVERLAP
    assert fwd(A1, n, v, v, A2, -100, 2, -1, A3, A4, None, A4, 1 << 20, None) == OVERLAP
    if _no_gpu():
        assert fwd(A1, n, v, v, A2, -100, 2, -1, A3, A5, A6, A4, 1 << 20, None) in AT_DEVICE_CHECK
    bwd = lib.ce_chunked_bwd
    # the gradient one row into the logits (same stride, different start): refused; exactly
    # the logits rows: the in-place case
    assert bwd(A1, n, v, v, A1 + 2 * v, v, A2, -100, 2, -1, None, None, None, A4, 1 << 20,
               None) == OVERLAP
    assert bwd(A1, n, v, 16, A1, 8, A2, -100, 2, -1, None, None, None, A4, 1 << 20,
               None) == OVERLAP  # same start, different row stride
    assert bwd(A1, n, v, v, A5, v, A2, -100, 2, -1, None, A5 + 8, None, A4, 1 << 20,
               None) == OVERLAP  # lse inside the gradient
    if _no_gpu():
        assert bwd(A1, n, v, v, A1, v, A2, -100, 2, -1, None, A3, None, A4, 1 << 20,
                   None) in AT_DEVICE_CHECK
        assert lib.ce_chunked_bwd_inplace(A1, n, v, v, A2, -100, 2, -1, None, A3, None, A4,
                                          1 << 20, None) in AT_DEVICE_CHECK
    fused = lib.ce_chunked_fwd_bwd_inplace
    assert fused(A1, n, v, v, A2, -100, 2, -1, None, A1 + 4, None, None, A4, 1 << 20,
                 None) == OVERLAP  # the loss inside the logits it overwrites
    assert fused(A1, n, v, v, A2, -100, 2, -1, A4 + 8, A3, None, None, A4, 1 << 20,
                 None) == OVERLAP  # the upstream gradient inside the workspace
    rows_f, rows_b = lib.ce_rows_fwd, lib.ce_rows_bwd
    assert rows_f(A1, n, v, v, A2, -100, 2, A2, None, None, A4, 1 << 20, None) == OVERLAP
    assert rows_b(A1, n, v, v, A5, v, A2, -100, 2, A5 + 4, None, None, A4, 1 << 20,
                  None) == OVERLAP  # grad_rows inside the gradient


def _flce_args(**kw):
    a = dict(hidden=A1, weight=A2, bias=None, labels=A3, n=4, h=16, v=10, ign=-100, chunk=2,
             t=-1, flags=0, gout=None, loss=A4, lse=None, gh=A5, gw=A6, gb=None, status=None,
             ws=A7, wsb=1 << 22, stream=None)
    a.update(kw)
    return list(a.values())


def test_flce_overlapping_buffers_are_refused(lib):
    f = lib.flce_fwd_bwd
    # grad_hidden as scratch: never the hidden rows (no in-place form), never another buffer
    assert f(*_flce_args(gh=A1)) == OVERLAP
    assert f(*_flce_args(gh=A1 + 64)) == OVERLAP
    assert f(*_flce_args(gh=A2 + 16)) == OVERLAP
    assert f(*_flce_args(gh=A3)) == OVERLAP
    assert f(*_flce_args(bias=A8, gh=A8)) == OVERLAP
    assert f(*_flce_args(gh=A7 + 256)) == OVERLAP     # inside the workspace
    assert f(*_flce_args(gw=A5 + 16 * 2)) == OVERLAP   # grad_weight over grad_hidden
    assert f(*_flce_args(ws=A2)) == OVERLAP            # the workspace over the weight
    assert f(*_flce_args(loss=A5 + 4)) == OVERLAP
    assert f(*_flce_args(lse=A1 + 4)) == OVERLAP
    assert f(*_flce_args(status=A6)) == OVERLAP
    assert f(*_flce_args(gout=A6 + 8)) == OVERLAP
    if _no_gpu():
        assert f(*_flce_args(bias=A8, gb=A9, lse=A10, status=A11, gout=A12)) in AT_DEVICE_CHECK
    fwd = lib.flce_fwd
    assert fwd(A1, A2, None, A3, 4, 16, 10, -100, 2, -1, A4, A1 + 8, None, A7, 1 << 22,
               None) == OVERLAP  # lse inside hidden
    bwd = lib.flce_bwd
    base = [A1, A2, None, A3, A4, 4, 16, 10, -100, 2, -1, 0, None, A5, A6, None, None, A7,
            1 << 22, None]
    if _no_gpu():
        assert bwd(*base) in AT_DEVICE_CHECK
    hit = list(base)
    hit[13] = A4  # grad_hidden over the saved lse
    assert bwd(*hit) == OVERLAP


def test_noalloc_step_argument_errors(lib):
    f = lib.ce_chunked_fwd_bwd_inplace_noalloc

    def call(logits=A1, n=4, v=8, ld=8, labels=A2, chunk=2, gout=None, loss=A3, lse=None,
             status=None):
        return f(logits, n, v, ld, labels, -100, chunk, -1, gout, loss, lse, status, None)

    assert call(n=-1) == BAD_SHAPE
    assert call(ld=7) == BAD_SHAPE
    assert call(chunk=0) == BAD_CHUNK
    assert call(loss=None) == NULL_ARG
    assert call(logits=A1 + 1) == ALIGN
    assert call(n=lce.LCE_NOALLOC_MAX_ROWS + 1) == SCRATCH_LIMIT
    assert call(loss=A1 + 4) == OVERLAP                           # the loss inside the logits
    if _no_gpu():
        assert call(n=lce.LCE_NOALLOC_MAX_ROWS, v=1, ld=1) in AT_DEVICE_CHECK
        assert call(lse=A4, status=A5, gout=A6) in AT_DEVICE_CHECK
