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

FEATS = [1, 1, 1, 2, 2, 3, 4, 5, 6, 7, 8, 9, 10, 12, 14, 16, 18, 24, 30, 31, 32, 32, 33, 34, 48, 63, 64, 64,
         65, 66, 96, 127, 128, 129, 130, 255, 256, 257, 258, 300, 513]
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
    # zipf_runs: Zipf-distributed run lengths
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


# ---------------------------------------------------------------- runs, scatter, search

def _keys(rng):
    """Keys with a random run structure; sizes often near the 4,096-key tiles."""
    n = int(rng.choice([int(rng.integers(0, 300_000)), 4096 * int(rng.integers(1, 40)) + int(rng.integers(-2, 3))]))
    n = max(n, 0)
    mix = int(rng.integers(0, 4))
    if mix == 0:  # short random runs
        lens = rng.integers(1, 8, n + 1)
    elif mix == 1:  # long runs
        lens = rng.integers(1, 20_000, n // 1000 + 2)
    elif mix == 2:  # all distinct
        lens = np.ones(n + 1, dtype=np.int64)
    else:  # Zipf run lengths
        lens = np.minimum(rng.zipf(1.3, n + 1), 100_000)
    vals = rng.integers(0, 2 ** 32, lens.size, dtype=np.uint32)
    if rng.random() < 0.3:  # few distinct keys: neighbouring runs may still differ only by run
        vals = rng.integers(0, 3, lens.size).astype(np.uint32)
    keys = np.repeat(vals, lens)[:n]
    return np.ascontiguousarray(keys, dtype=np.uint32)


@pytest.mark.parametrize("seed", range(60))
def test_runs_fuzz(seed):
    import segmented_reduction_amd as sr
    import oracle
    rng = np.random.default_rng(0x5EED + seed)
    keys = _keys(rng)
    gu.say(f"fuzz runs seed={seed} n={keys.size}")
    v, ln, off, c = sr.rle(gu.to_gpu(keys))
    ov, oln, ooff, oc = oracle.rle(keys)
    assert c == oc
    assert np.array_equal(v.cpu().numpy(), ov) and np.array_equal(ln.cpu().numpy(), oln)
    assert np.array_equal(off.cpu().numpy(), ooff)
    uv, uc = sr.unique(gu.to_gpu(keys))
    uc = int(uc.item())
    wv, wc = oracle.unique(keys)
    assert uc == wc and np.array_equal(uv[:uc].cpu().numpy(), wv)
    flags = (rng.random(keys.size) < rng.choice([0.001, 0.1, 0.5, 0.99])).astype(np.uint32)
    flags[flags == 1] = rng.integers(1, 2 ** 32, int(flags.sum()), dtype=np.uint32)  # any nonzero marks a start
    fo, fc = sr.offsets_from_flags(gu.to_gpu(flags))
    fc = int(fc.item())
    wo, wc = oracle.offsets_from_flags(flags)
    assert fc == wc and np.array_equal(fo[: fc + 1].cpu().numpy(), wo)


@pytest.mark.parametrize("seed", range(80))
def test_scatter_fuzz(seed):
    import workloads as W
    from tests.test_gpu_scatter import _check as scatter_check
    rng = np.random.default_rng(0x5CA7 + seed)
    kind = ["u32", "i32", "f32"][int(rng.integers(0, 3))]
    feat = [1, 1, 2, 3, 4, 7, 8, 9, 16, 31, 32, 33, 64, 65, 100, 200][int(rng.integers(0, 16))]
    rows = int(rng.integers(0, max(2, 600_000 // feat)))
    dim = int(rng.choice([1, 2, 3, 7, 100, 1000, 4096, 20_000, 300_000]))
    order = ["random", "sorted", "runs", "one"][int(rng.integers(0, 4))]
    oor = float(rng.choice([0.0, 0.0, 0.01, 0.3]))
    values = "ties" if rng.random() < 0.3 else "normal"
    index, vals = W.scatter_case(int(rng.integers(0, 2 ** 31)), rows, dim, feat=feat, dtype=kind, order=order,
                                 out_of_range=oor, values=values)
    ops = ["sum", "min", "max"] + (["mean"] if kind == "f32" else [])
    op = ops[int(rng.integers(0, len(ops)))]
    scatter_check(index, vals, dim, op, what=f"fuzz seed={seed} F={feat} {order} oor={oor} {values}")


@pytest.mark.parametrize("seed", range(30))
def test_index_offsets_fuzz(seed):
    import segmented_reduction_amd as sr
    import oracle
    import workloads as W
    import torch
    rng = np.random.default_rng(0x1DE + seed)
    rows = int(rng.integers(0, 400_000))
    dim = int(rng.choice([0, 1, 5, 4095, 4096, 4097, 50_000, 500_000]))
    order = ["sorted", "runs", "random"][int(rng.integers(0, 3))]
    index, _ = W.scatter_case(int(rng.integers(0, 2 ** 31)), rows, dim, feat=1, order=order,
                              out_of_range=float(rng.choice([0.0, 0.05])))
    gu.say(f"fuzz offsets_from_index seed={seed} rows={rows} dim={dim} {order}")
    got = sr.offsets_from_index(gu.to_gpu(index), dim)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.offsets_from_index(index, dim))


@pytest.mark.parametrize("seed", range(40))
def test_search_fuzz(seed):
    from tests.pins import _lb_case
    from tests.test_gpu_search import _check as search_check
    rng = np.random.default_rng(0x5EA + seed)
    kind = ["u32", "f32"][seed % 2]
    segs = int(rng.integers(1, 300))
    vmax = int(rng.choice([0, 1, 5, 64, 700, 5000]))
    qmax = int(rng.choice([0, 1, 7, 33, 300, 2049]))
    tile = int(rng.choice([1, 2, 5, 32, 64, 100, 256]))
    use_order = bool(rng.random() < 0.3)
    stride = 1 if use_order else int(rng.choice([1, 1, 2, 5]))
    stored, qs, seg, ordv, pool = _lb_case(rng, kind, segs, vmax, qmax, order=use_order, stride=stride)
    kw = dict(tile=tile)
    if use_order:
        kw["order"] = ordv
    if stride > 1:
        kw["stride"] = stride
        kw["value_count"] = pool.shape[0]
    search_check(stored, qs, seg, what=f"fuzz seed={seed}", **kw)
