"""Buffer-descriptor ranges of the streaming kernels, replayed on the host.

Every read of `values` (and every write of the scan's `out`) goes through a
raw buffer descriptor whose range the hardware checks against the lane
offset (VGPR offset plus immediate); accesses at or past the range return 0
or are dropped.  So no byte past the valid rows is touched as long as every
descriptor the kernels build lies inside [offsets[0] * F * 4,
offsets[S] * F * 4).  This test rebuilds, with the kernels' own expressions,
every descriptor each kernel can form -- for every share of several share
counts, every chunk or batch start inside the share and every feature
block -- on inputs whose last row ends the allocation, and checks that.
(The expressions are copied from the kernel sources by hand; a change there
must be mirrored here.)"""
import numpy as np
import pytest

import workloads as W

FEATS = [1, 2, 3, 4, 5, 6, 8, 10, 12, 14, 16, 18, 24, 30, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 260]


def _shares(off, nw, cw=1, gran=1, min_share=1, period=0):
    """Merge-path shares (d0, d1, i0, j0, i1, j1), rows relative to off[0];
    with a period, share sizes within period / 16 of a multiple of it grow
    to the band's edge."""
    o0 = int(off[0])
    s = len(off) - 1
    keys = off - o0 + cw * np.arange(s + 1)
    t = int(keys[-1])  # rows + cw * S
    dg = max(-(-t // (nw * gran)), -(-min_share // gran))
    d = dg * gran
    if period > 0 and d >= period:
        m, r = period // 16, d % period
        if r < m:
            d += m - r
        elif r > period - m:
            d += period - r + m
        d = -(-d // gran) * gran

    def at(diag):
        i = int(np.searchsorted(keys, diag, side="right")) - 1
        j = diag - cw * i
        if cw != 1 and i < s:
            j = min(j, int(off[i + 1]) - o0)
        return i, j

    out = []
    for w in range(nw):
        d0, d1 = min(w * d, t), min(w * d + d, t)
        (i0, j0), (i1, j1) = at(d0), at(d1)
        out.append((d0, d1, i0, j0, i1, j1, d))
    return out


def _check(lo_byte, hi_byte, base_elems, size_bytes, what):
    if size_bytes == 0:
        return
    assert base_elems * 4 >= lo_byte, what
    assert base_elems * 4 + size_bytes <= hi_byte, (what, base_elems * 4 + size_bytes, hi_byte)
    assert size_bytes < 2 ** 32, what


@pytest.mark.parametrize("feat", FEATS)
def test_descriptors_stay_inside_the_rows(feat):
    off, _ = W.ragged(seed=feat, segments=300, mean_len=7, feat=1, empty_frac=0.2, base=3, long_segment=900)
    off = off.astype(np.int64)
    o0, n_end = int(off[0]), int(off[-1])
    lo, hi = o0 * feat * 4, n_end * feat * 4  # the valid rows; the allocation ends at hi
    for nw in (4, 12, 64, 400):
        if feat == 1:
            # seg_reduce_flat: chunk of CH = 2048 elements from row jc, descriptor
            # make_rsrc(values + (o0 + jc), rmax * 4), rmax = min(CH, j1 - jc)
            for _, _, _, j0, _, j1, _ in _shares(off, nw, cw=8, min_share=2048):
                for jc in range(j0, j1 + 1):
                    rmax = min(2048, j1 - jc)
                    _check(lo, hi, o0 + jc, rmax * 4, ("flat", nw, jc))
            # seg_scan tails (1-D): batch of E = 64 * 4 * U (U = 4) from rb,
            # make_rsrc(values + o0 + rb, n * 4), n = max(0, min(E, j1 - rb))
            for _, _, _, j0, _, j1, _ in _shares(off, nw):
                for rb in range(j0, j1 + 1):
                    n = max(0, min(1024, j1 - rb))
                    _check(lo, hi, o0 + rb, n * 4, ("scan tails 1-D", nw, rb))
        row_bytes = feat * 4
        vec4 = feat % 4 == 0
        if feat == 32:
            # seg_reduce_team (rows of 32 features, 16-byte access): one
            # descriptor over the wave's share, from
            # feature block fbase: make_rsrc(values + (o0 + j0) * F + fbase,
            # (j1 - j0) * F * 4 - fbase * 4)
            units = feat // 4 if vec4 else feat
            lanes = 1 if vec4 else 2
            while lanes < units and lanes < 64:
                lanes *= 2
            fb = lanes * (4 if vec4 else 1)
            for _, _, _, j0, _, j1, _ in _shares(off, nw, gran=64 // lanes, period=65536 // (feat * 4)):
                for fbase in range(0, feat, fb):
                    size = (j1 - j0) * feat * 4 - fbase * 4 if j1 > j0 else 0
                    _check(lo, hi, (o0 + j0) * feat + fbase, size, ("team", nw, fbase))
        if feat > 1:
            # seg_reduce_rows: chunk of CH rows from row jc and feature block
            # fbase, make_rsrc(values + (o0 + jc) * F + fbase, rmax * row_bytes - fbase * 4)
            for vec, lanes in ((4, min(64, 1 << (max(1, feat // 4) - 1).bit_length())),
                               (2, min(64, 1 << (max(1, feat // 2) - 1).bit_length())),
                               (1, min(64, 1 << (feat - 1).bit_length()))):
                if vec == 4 and not vec4 or vec == 2 and (vec4 or feat % 2):
                    continue
                lanes = max(lanes, 1 if vec > 1 else 2)
                # rows per group (rows of fewer than 32 features are read
                # through LDS, 1 KB per load instruction: the same bytes of
                # the same descriptor)
                if vec == 4:
                    v = 8
                elif vec == 2:
                    v = 16 if feat in (2, 6) or lanes in (8, 16) else 8
                else:
                    v = 32 if lanes <= 32 else 24
                ch = (64 // lanes) * v
                for _, _, _, j0, _, j1, _ in _shares(off, nw):
                    for jc in range(j0, j1 + 1):
                        rmax = min(ch, j1 - jc)
                        for fbase in range(0, feat, lanes * vec):
                            size = rmax * row_bytes - fbase * 4 if rmax > 0 else 0
                            _check(lo, hi, (o0 + jc) * feat + fbase, size, ("rows", vec, nw, jc, fbase))
            # seg_scan tails (rows): make_rsrc(values + (o0 + rb) * F + chunk * 64,
            # n * F * 4 - chunk * 64 * 4), n = max(0, min(E, j1 - rb))
            lanes = min(64, 1 << (feat - 1).bit_length())
            e = (64 // lanes) * 16
            for _, _, _, j0, _, j1, _ in _shares(off, nw):
                for rb in range(j0, j1 + 1, max(1, (j1 - j0) // 50)):
                    n = max(0, min(e, j1 - rb))
                    for chunk in range(0, -(-feat // 64)):
                        size = (n * feat - chunk * 64) * 4 if n > 0 else 0
                        _check(lo, hi, (o0 + rb) * feat + chunk * 64, size, ("scan tails", nw, rb, chunk))
        # seg_scan main: batch of B = U * SR rows from rb0 and feature block
        # fbase, make_rsrc(values + (o0 + rb0) * F + fbase, (nrows * F - fbase) * 4)
        # (the same range for `out`), nrows = min(B, j1 - rb0)
        lanes = 1 if feat == 1 else min(64, 1 << (feat - 1).bit_length())
        vv = 4 if feat == 1 else 1
        b = (16 if vv == 1 else 4) * (64 // lanes) * vv
        for _, _, _, j0, _, j1, _ in _shares(off, nw):
            for rb0 in range(j0, j1 + 1, max(1, (j1 - j0) // 50)):
                nrows = min(b, j1 - rb0)
                for fbase in range(0, feat, 64 if feat > 1 else 1):
                    size = (nrows * feat - fbase) * 4 if nrows > 0 else 0
                    _check(lo, hi, (o0 + rb0) * feat + fbase, size, ("scan main", nw, rb0, fbase))


def test_the_old_row_descriptor_would_fail():
    """The check catches the range the row kernel used to give its chunk
    descriptors (rmax * row_bytes from the feature block's first feature)."""
    off = np.array([0, 5, 9], dtype=np.int64)
    feat, fbase, jc, rmax = 100, 64, 0, 9
    with pytest.raises(AssertionError):
        _check(0, 9 * feat * 4, jc * feat + fbase, rmax * feat * 4, "old")
    _check(0, 9 * feat * 4, jc * feat + fbase, rmax * feat * 4 - fbase * 4, "new")
    assert off[-1] == 9
