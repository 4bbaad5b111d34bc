"""Seeded random sweep of the segmented reduction and scan against the CPU
oracle (GPU only).

Each case draws a dtype, an operation, a row width around the kernels' class
boundaries (1-D, rows of at most 128 bytes, wider rows, rows wider than one
256-feature block), a segment-length mix (uniform, heavy-tailed, all ones,
long runs of empty segments, a few huge segments among short ones), value
kinds (normal / wide integers, few distinct values for ties, small integers
as floats, and for min/max the float specials: signed zeros, infinities,
NaN bit patterns, denormals), a first offset above zero, unread rows after
the last offset, and a work partition (the default or a forced share
count).  Integer results, min/max values and rows must match the oracle bit
for bit, float sums within 1e-5 * sum|x| + 1e-6 (means: that bound over the
length), scans as in the scan tests."""
import numpy as np
import pytest

from tests import gpu_util as gu
from tests.test_gpu_scan import _check as scan_check

pytestmark = pytest.mark.gpu

FEATS = [1, 1, 1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 24, 31, 32, 32, 33, 48, 63, 64, 64, 65, 96, 127, 128, 129,
         255, 256, 257, 300, 513]
MIXES = ["uniform", "pareto", "ones", "empty_runs", "few_huge", "zipf_runs"]
SHARES = [None, None, None, 1, 2, 3, 4, 7, 64, 333, 4096, 5000]


@pytest.fixture(autouse=True)
def _reset_shares():
    import segmented_reduction_amd as sr
    sr.set_shares(0)
    yield
    sr.set_shares(0)


def _lengths(rng, mix, segs, mean):
    if mix == "uniform":
        return rng.integers(0, 2 * mean + 1, segs)
    if mix == "pareto":
        return np.minimum((rng.pareto(1.5, segs) * mean / 2).astype(np.int64), 50 * mean + 1)
    if mix == "ones":
        return np.ones(segs, dtype=np.int64)
    if mix == "empty_runs":
        ln = rng.integers(1, 2 * mean + 1, segs)
        for _ in range(max(1, segs // 200)):
            a = int(rng.integers(0, segs))
            ln[a:a + int(rng.integers(1, 400))] = 0
        return ln
    if mix == "few_huge":
        ln = rng.integers(0, 4, segs)
        for _ in range(int(rng.integers(1, 4))):
            ln[int(rng.integers(0, segs))] = int(rng.integers(20 * mean, 200 * mean + 1))
        return ln
    # zipf_runs: run lengths of a sorted Zipf sample, in random order
    ln = np.minimum(rng.zipf(1.6, segs), 100 * mean + 1)
    return ln.astype(np.int64)


_SPECIAL_BITS = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001,
                          0x00000001, 0x80000001, 0x007FFFFF, 0x7F7FFFFF, 0xFF7FFFFF, 0x3F800000, 0xBF800000],
                         dtype=np.uint32)


def _values(rng, kind, vkind, shape):
    if vkind == "ties":
        v = rng.integers(-2, 3, shape)
        return {"f32": (v * 0.5).astype(np.float32), "i32": v.astype(np.int32), "u32": (v + 2).astype(np.uint32)}[kind]
    if vkind == "intfloat" and kind == "f32":
        return rng.integers(-3, 4, shape).astype(np.float32)
    if vkind == "special" and kind == "f32":
        bits = rng.integers(0, 2 ** 32, shape, dtype=np.uint32)
        pick = rng.random(shape) < 0.5
        bits[pick] = _SPECIAL_BITS[rng.integers(0, _SPECIAL_BITS.size, int(pick.sum()))]
        return bits.view(np.float32)
    if kind == "f32":
        return rng.standard_normal(shape, dtype=np.float32)
    if kind == "i32":
        return rng.integers(-(2 ** 31), 2 ** 31, shape, dtype=np.int32)
    return rng.integers(0, 2 ** 32, shape, dtype=np.uint32)


def _case(seed):
    rng = np.random.default_rng(0xF5A + seed)
    kind = ["u32", "i32", "f32", "f32"][int(rng.integers(0, 4))]
    feat = FEATS[int(rng.integers(0, len(FEATS)))]
    ops = ["sum", "min", "max"] + (["mean"] if kind == "f32" else [])
    op = ops[int(rng.integers(0, len(ops)))]
    mix = MIXES[int(rng.integers(0, len(MIXES)))]
    budget = 400_000 if feat == 1 else max(2_000, 1_500_000 // feat)  # rows
    mean = int(rng.integers(1, 80))
    segs = int(rng.integers(1, max(2, budget // (mean + 1))))
    ln = _lengths(rng, mix, segs, mean)
    if ln.sum() > budget:  # keep the oracle quick
        ln = (ln * (budget / ln.sum())).astype(np.int64)
    base = int(rng.integers(0, 40))
    tail = int(rng.integers(0, 40))
    off = np.zeros(segs + 1, dtype=np.int64)
    off[0] = base
    np.cumsum(ln, out=off[1:])
    off[1:] += base
    rows = int(off[-1]) + tail
    vkinds = ["normal", "ties", "intfloat"] + (["special"] if op in ("min", "max") else [])
    vkind = vkinds[int(rng.integers(0, len(vkinds)))]
    shape = (rows,) if feat == 1 else (rows, feat)
    vals = _values(rng, kind, vkind, shape)
    shares = SHARES[int(rng.integers(0, len(SHARES)))]
    return vals, off, op, shares, f"fuzz seed={seed} kind={kind} F={feat} mix={mix} values={vkind}"


@pytest.mark.parametrize("seed", range(400))
def test_reduce_fuzz(seed):
    vals, off, op, shares, what = _case(seed)
    gu.check(vals, off, op, shares=shares, what=what)


@pytest.mark.parametrize("seed", range(400, 600))
def test_scan_fuzz(seed):
    vals, off, op, shares, what = _case(seed)
    if op == "mean":  # the scan has no mean
        op = "sum"
    exclusive = bool(seed % 2)
    scan_check(vals, off, op, exclusive, shares=shares, what=what)


def test_fuzz_cases_are_valid():
    """The generator keeps offsets nondecreasing and inside the rows."""
    for seed in range(600):
        vals, off, op, shares, _ = _case(seed)
        assert (np.diff(off) >= 0).all() and off[0] >= 0 and off[-1] <= vals.shape[0]
        if op in ("sum", "mean") and vals.dtype == np.float32:
            assert np.isfinite(vals).all()  # specials only where no tolerance is needed
