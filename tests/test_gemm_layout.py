"""Host checks of the pipelined GEMM's index arithmetic (no GPU).

The kernel's LDS layouts, DMA placement and fragment reads are restated here from their
definitions in ``csrc/gemm_tile.h`` and checked against each other: every byte a slice's DMA
writes lands in a distinct place, and every MFMA fragment read returns the elements the
MFMA expects. The lane order of ``ds_read_b64_tr_b16`` used below (lane i of each 16-lane
group receives element i mod 4 of the 8-byte reads of lanes 4e + i/4, e = 0..3) was measured
on the device. Also checked: the XCD-block tile mapping covers every tile once, and the
slice window steps of grouped K-major operands.
"""
import pytest


def swz_k(bk, r):
    return (r & 7) if bk == 64 else ((r >> 1) & 3)


def swz_mn(k):
    return 2 * ((k & 3) | ((k >> 1) & 4))


def place_slice(kmajor, rows, bk, nw):
    """LDS 16-byte chunk -> (kind, row or k, first element) written by one slice's DMA."""
    per = rows * bk * 2 // 1024 // nw
    assert per * nw * 1024 == rows * bk * 2
    lds = {}
    for w in range(nw):
        for j in range(per):
            g = w * per + j
            for l in range(64):
                dst = g * 1024 + 16 * l
                if kmajor:
                    kc = bk // 8
                    r = (64 // kc) * g + l // kc
                    c = (l % kc) ^ swz_k(bk, r)
                    src = ("K", r, 8 * c)
                else:
                    rc = rows // 8
                    k = (64 // rc) * g + l // rc
                    c = (l % rc) ^ swz_mn(k)
                    src = ("M", k, 8 * c)
                assert dst not in lds
                lds[dst] = src
    assert len(lds) * 16 == rows * bk * 2
    return lds


def element(lds, addr):
    kind, a, b = lds[addr - addr % 16]
    return kind, a, b + (addr % 16) // 2


@pytest.mark.parametrize("kmajor,rows,bk,nw", [
    (True, 256, 64, 8), (False, 256, 64, 8), (True, 256, 32, 4), (False, 256, 32, 4),
    (False, 128, 32, 4), (True, 128, 32, 4)])
def test_dma_placement_matches_fragment_reads(kmajor, rows, bk, nw):
    lds = place_slice(kmajor, rows, bk, nw)
    for rbase in range(0, rows, 16):
        for kk in range(bk // 32):
            for l in range(64):
                if kmajor:
                    r = rbase + (l & 15)
                    c = (4 * kk + (l >> 4)) ^ swz_k(bk, r)
                    got = [element(lds, r * 2 * bk + c * 16 + 2 * e) for e in range(8)]
                    want = [("K", r, 32 * kk + 8 * (l >> 4) + e) for e in range(8)]
                else:
                    def read8(lane):
                        ll = lane & 15
                        m = rbase + 4 * (ll & 3)
                        k0 = 32 * kk + 8 * (lane >> 4) + (ll >> 2)
                        c = m >> 3
                        half = ((m >> 2) & 1) * 8
                        return [[element(lds, kx * 2 * rows + ((c ^ swz_mn(kx)) << 4) + half + 2 * e)
                                 for e in range(4)] for kx in (k0, k0 + 4)]
                    lo = l & 15
                    got = [read8((l & 48) + 4 * e + lo // 4)[half][lo % 4]
                           for half in range(2) for e in range(4)]
                    want = [("M", 32 * kk + 8 * (l >> 4) + e, rbase + lo) for e in range(8)]
                assert got == want


def xcd_blocks(mt, nt):
    xn = 4 if nt % 4 == 0 else (2 if nt % 2 == 0 else 1)
    gm = 8 // xn
    grid = 8 * ((mt + gm - 1) // gm) * (nt // xn)
    seen = set()
    for w in range(grid):
        x, li = w & 7, w >> 3
        xm, xq = x // xn, x % xn
        m_lo, m_hi = xm * mt // gm, (xm + 1) * mt // gm
        n_lo, n_hi = xq * nt // xn, (xq + 1) * nt // xn
        nn = n_hi - n_lo
        if nn <= 0 or li >= (m_hi - m_lo) * nn:
            continue
        t = (m_lo + li // nn, n_lo + li % nn)
        assert 0 <= t[0] < mt and 0 <= t[1] < nt and t not in seen
        seen.add(t)
    assert len(seen) == mt * nt


@pytest.mark.parametrize("mt", [8, 9, 15, 129, 501])
@pytest.mark.parametrize("nt", [1, 2, 3, 6, 16, 32, 33])
def test_xcd_block_mapping_covers_every_tile_once(mt, nt):
    xcd_blocks(mt, nt)


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("k0", [0, 32, 64, 96, 448])
def test_grouped_kmajor_window_steps(gs, k0):
    """32-deep slices of a K-major operand stored in 64-column groups gs elements apart:
    the window advances 32 elements, then to the next group's start."""
    def start(k):
        return ((k >> 6) * gs + (k & 63)) * 2
    base = start(k0)
    step, step2 = ((gs - 32) * 2, 64) if (k0 & 32) else (64, (gs - 32) * 2)
    for n in range(1, 20):
        base += step
        step, step2 = step2, step
        assert base == start(k0 + 32 * n)
