"""Invariants of the seeded input generators (CPU only)."""
import numpy as np

import workloads as W


def test_small_shape():
    c = W.small()
    off = c["offsets"]
    assert off.shape == (4097,) and off[0] == 0 and (np.diff(off) >= 0).all()
    assert np.diff(off).max() <= 64
    assert 0.02 < (np.diff(off) == 0).mean() < 0.045
    assert c["f32"].shape == c["i32"].shape == (off[-1],)
    assert c["i32"].min() >= -1000 and c["i32"].max() <= 1000


def test_small_is_seeded():
    a, b = W.small(0), W.small(0)
    assert np.array_equal(a["f32"], b["f32"]) and np.array_equal(a["offsets"], b["offsets"])
    assert not np.array_equal(a["offsets"], W.small(1)["offsets"])


def test_message_shape():
    c = W.message()
    off = c["offsets"]
    assert off.shape == (10_001,) and off[-1] == 1_000_000
    assert c["f32"].shape == (1_000_000, 64) and c["f32"].dtype == np.float32
    assert abs(np.diff(off).mean() - 100) < 1e-9


def test_skew_shape():
    c = W.skew(values=False)
    d = np.diff(c["offsets"])
    assert c["offsets"][-1] == 50_000_000 and d.size == 1_000_000
    assert (d == 0).sum() == 100_000 and d.max() == 5_000_000 and d[c["hub"]] == 5_000_000


def test_powerlaw_shape():
    c = W.powerlaw(values=False)
    d = np.diff(c["offsets"])
    assert c["offsets"][-1] == 32_000_000 and d.size == 2_000_000
    assert d.max() == 200_000 and d[c["hub"]] == 200_000
    assert 0.09 < (d == 0).mean() < 0.13


def test_rle_keys_sorted_zipf():
    c = W.rle_keys(n=1_000_000)
    k = c["keys"]
    assert k.dtype == np.uint32 and (k[1:] >= k[:-1]).all()
    assert k.max() < 2 ** 20
    _, counts = np.unique(k, return_counts=True)
    # the most frequent key carries roughly 1 / zeta-like share of the draws
    assert counts.max() > 0.08 * k.size


def test_ragged_case():
    off, v = W.ragged(3, 50, 10, feat=3, dtype="u32", base=7, tail_rows=2, long_segment=100)
    assert off[0] == 7 and v.shape == (off[-1] + 2, 3) and v.dtype == np.uint32
    assert np.diff(off).max() == 100


def test_scatter_shape():
    c = W.scatter()
    idx = c["index"]
    assert idx.shape == (1_000_000,) and idx.dtype == np.int64 and c["dim"] == 10_000
    assert idx.min() >= 0 and idx.max() < 10_000 and not (np.diff(idx) >= 0).all()  # unsorted
    assert abs(np.bincount(idx, minlength=10_000).mean() - 100) < 1e-9
    assert c["f32"].shape == (1_000_000, 64) and c["f32"].dtype == np.float32


def test_scatter_case_orders():
    idx, v = W.scatter_case(3, 5000, 300, feat=2, order="sorted", out_of_range=0.1)
    inr = idx[(idx >= 0) & (idx < 300)]
    assert (np.diff(inr) >= 0).all() and v.shape == (5000, 2)
    assert 0.05 < ((idx < 0) | (idx >= 300)).mean() < 0.15
    idx, _ = W.scatter_case(4, 5000, 300, order="runs")
    assert (np.diff(idx) == 0).mean() > 0.8
    idx, _ = W.scatter_case(5, 100, 7, order="one")
    assert (idx == 0).all()


def test_search_shape():
    c = W.search()
    v, q, seg = c["values"], c["queries"], c["segments"]
    assert seg.shape == (8192, 4) and seg.dtype == np.int64
    assert v.dtype == np.float32 and q.dtype == np.float32
    assert seg[:, 1].sum() == v.size and seg[:, 3].sum() == q.size and seg[:, 3].max() <= 2049
    for vo, vc, qo, qc in seg[::97]:
        assert (np.diff(v[vo:vo + vc]) >= 0).all() and (np.diff(q[qo:qo + qc]) >= 0).all()
        if vc:
            assert v[vo] > 0
