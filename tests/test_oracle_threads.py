"""The oracle on several host threads (the benchmark's CPU baseline) gives
exactly the single-thread results: each thread takes a contiguous range of
segments and reduces each segment in one sequential pass."""
import numpy as np
import pytest

import oracle
import workloads as W


@pytest.mark.parametrize("feat,kind", [(1, "f32"), (8, "f32"), (3, "i32"), (1, "u32")])
def test_threads_do_not_change_results(feat, kind):
    off, vals = W.ragged(seed=feat + 11, segments=5000, mean_len=25, feat=feat, dtype=kind, base=4,
                         long_segment=20000)
    for op in ("sum", "min", "max") + (("mean",) if kind == "f32" else ()):
        one = oracle.reduce(vals, off, op)
        for t in (2, 3, 7, 16):
            many = oracle.reduce(vals, off, op, threads=t)
            assert np.array_equal(one.out.view(np.uint32), many.out.view(np.uint32)), (op, t)
            if one.arg is not None:
                assert np.array_equal(one.arg, many.arg), (op, t)
            if one.ref is not None:
                assert np.array_equal(one.ref, many.ref) and np.array_equal(one.mag, many.mag), (op, t)


def test_segment_ranges_cover_every_segment_once():
    off, _ = W.ragged(seed=3, segments=1000, mean_len=10, base=7, long_segment=5000)
    for parts in (1, 2, 5, 64, 2000):
        rs = oracle.segment_ranges(off, parts)
        assert rs[0][0] == 0 and rs[-1][1] == len(off) - 1
        assert all(a < b for a, b in rs) and all(rs[i][1] == rs[i + 1][0] for i in range(len(rs) - 1))
