"""Parity of the HIP lower-bound search (segred_galloping_search) with the
CPU oracle, bit for bit: positions, validation word, and untouched outputs
(GPU only)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_util as gu
from tests.pins import _lb_case

pytestmark = pytest.mark.gpu

UNSET = -7


def _gpu(stored, qs, seg, *, stride=1, order=None, value_count=None, max_qc=None, tile=32, word=0, preserve=False):
    import segmented_reduction_amd as sr
    v, q = gu.to_gpu(stored), gu.to_gpu(qs)
    sg = gu.to_gpu(np.ascontiguousarray(seg, dtype=np.int64).reshape(-1, 4))
    o = gu.to_gpu(order) if order is not None else None
    out = torch.full((max(qs.shape[0], 1),), UNSET, dtype=torch.int64, device="cuda")[: qs.shape[0]]
    val = torch.tensor([word], dtype=torch.int64).to(torch.int32).view(torch.uint32).cuda()
    if max_qc is None:
        max_qc = int(seg[:, 3].max()) if len(seg) else 0
    out, val = sr.galloping_search(v, q, sg, value_order=o, value_stride=stride, value_count=value_count,
                                   max_query_count=max_qc, queries_per_tile=tile, out=out, validation=val,
                                   preserve_validation=preserve)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(val.cpu().view(torch.int32).item()) & 0xFFFFFFFF


def _check(stored, qs, seg, what="", **kw):
    seg = np.ascontiguousarray(seg, dtype=np.int64).reshape(-1, 4)
    gu.say(f"search {what} dtype={gu.kind_of(stored)} values={stored.shape[0]} queries={qs.shape[0]} "
           f"S={seg.shape[0]} {kw.get('tile', 32)=} order={kw.get('order') is not None} stride={kw.get('stride', 1)}")
    got, word = _gpu(stored, qs, seg, **kw)
    okw = dict(kw)
    okw["out"] = np.full(qs.shape[0], UNSET, dtype=np.int64)
    okw["validation"] = okw.pop("word", 0)
    if "max_qc" not in okw or okw["max_qc"] is None:
        okw["max_qc"] = int(seg[:, 3].max()) if len(seg) else 0
    want, wword = oracle.lower_bounds(stored, qs, seg, **okw)
    assert word == wword, (what, word, wword)
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)[:5]
        raise AssertionError(f"{what}: positions differ at {bad.tolist()}: gpu {got[bad].tolist()} "
                             f"oracle {want[bad].tolist()}")


@pytest.mark.parametrize("kind", ["u32", "f32"])
@pytest.mark.parametrize("tile", [1, 5, 32, 100])
def test_random_segments(kind, tile):
    rng = np.random.default_rng(tile * 7 + (kind == "f32"))
    for trial in range(4):
        stored, qs, seg, _, _ = _lb_case(rng, kind, 40, 400, 300)
        _check(stored, qs, seg, what=f"random {trial}", tile=tile)


@pytest.mark.parametrize("kind", ["u32", "f32"])
def test_order_vector_and_stride(kind):
    rng = np.random.default_rng(5 + (kind == "f32"))
    stored, qs, seg, ordv, pool = _lb_case(rng, kind, 30, 500, 200, order=True)
    _check(stored, qs, seg, what="order", order=ordv)
    stored, qs, seg, _, pool = _lb_case(rng, kind, 30, 500, 200, stride=3)
    _check(stored, qs, seg, what="stride", stride=3, value_count=pool.shape[0])


def test_long_gallops():
    """Few, far-apart queries over long segments: gallops cross several
    coarse rounds; queries before, between and after all values; runs of
    duplicates."""
    rng = np.random.default_rng(11)
    v = np.sort(rng.integers(0, 2 ** 31, 3_000_000)).astype(np.uint32)
    v[1_000_000:1_200_000] = v[1_000_000]
    q = np.sort(np.concatenate([rng.integers(0, 2 ** 31, 300), [0, 0, v[1_000_000], v[-1], 2 ** 32 - 1]])).astype(np.uint32)
    m = q.size
    q2 = np.concatenate([q, q])  # each segment owns its own query range
    seg = np.array([[0, v.size, 0, m], [500_000, 1_500_000, m, m]])
    for tile in (3, 32, 400):
        _check(v, q2, seg, what="long", tile=tile)
    vf = np.sort(rng.standard_normal(2_000_000)).astype(np.float32)
    qf = np.sort(rng.standard_normal(257) * 1.5).astype(np.float32)
    _check(vf, qf, np.array([[0, vf.size, 0, qf.size]]), what="long f32", tile=16)


def test_validation_word():
    v = np.arange(10, dtype=np.float32)
    q = np.array([2.5, 1.0, 7.0, 3.0, np.nan, 4.0, 5.0, 8.0, 9.5, np.inf], dtype=np.float32)
    _check(v, q[:4], np.array([[0, 10, 0, 4]]), what="decrease", tile=4)
    _check(v, q[:2], np.array([[0, 10, 0, 2]]), what="decrease across tiles", tile=1)
    _check(v, q[3:10], np.array([[0, 10, 0, 7]]), what="non-finite", tile=3)
    _check(v, q[:3], np.array([[5, 6, 0, 3]]), what="value range")
    _check(v, q[:3], np.array([[0, 10, 1, 3]]), what="query range")
    _check(v, q[:3], np.array([[0, 10, 0, 3]]), what="capacity", max_qc=2)
    _check(v, q[:3], np.array([[-1, 2, 0, 3], [0, 10, 0, 1]]), what="negative offset")
    _check(v, q[:1], np.array([[4, 0, 0, 1], [0, 0, 1, 0]]), what="empty segments", word=16)
    _check(v, q[:2], np.array([[0, 10, 0, 2]]), what="preserve", tile=2, word=16, preserve=True)
    vu = np.array([1, 5, 0x80000000, 0xFFFFFFFF], dtype=np.uint32)
    _check(vu, np.array([0x7FFFFFFF, 0xFFFFFFFF], np.uint32), np.array([[0, 4, 0, 2]]), what="unsigned")


def test_decreasing_and_nonfinite_in_bulk():
    rng = np.random.default_rng(23)
    stored, qs, seg, _, _ = _lb_case(rng, "f32", 50, 300, 200)
    qs = qs.copy()
    idx = rng.choice(qs.shape[0], 40, replace=False)
    qs[idx[:25]] = rng.standard_normal(25).astype(np.float32)  # out of order
    qs[idx[25:]] = np.array([np.nan, np.inf, -np.inf] * 5, dtype=np.float32)
    _check(stored, qs, seg, what="bulk diagnostics", tile=8)


def test_many_queries_per_record():
    """Records with more queries than one staging batch (4,096): answered
    query by query, and with a NaN past that batch, tile by tile (the NaN's
    tile stops there, bit 8)."""
    rng = np.random.default_rng(31)
    v = np.sort(rng.standard_normal(3000)).astype(np.float32)
    q = np.concatenate([np.sort(rng.standard_normal(6000) * 1.2), np.sort(rng.standard_normal(4500))]).astype(np.float32)
    seg = np.array([[0, 3000, 0, 6000], [100, 2500, 6000, 4500]])  # query ranges must not overlap
    _check(v, q, seg, what="many queries", tile=32)
    q2 = q.copy()
    q2[4600] = np.nan
    q2[6000 + 4200] = np.inf
    _check(v, q2, seg, what="many queries, NaN past the batch", tile=32)
    vu = np.sort(rng.integers(0, 2 ** 32, 5000, dtype=np.uint64)).astype(np.uint32)
    qu = np.sort(rng.integers(0, 2 ** 32, 9000, dtype=np.uint64)).astype(np.uint32)
    _check(vu, qu, np.array([[0, 5000, 0, 9000], [7, 4000, 9000, 0]]), what="many queries u32, 5,000 values",
           tile=64)


def test_search_config_full_size():
    """The bench's workload at full size: every answer satisfies the lower
    bound property on the sorted segments (any size), and 96 sampled segments
    equal the oracle exactly."""
    import segmented_reduction_amd as sr
    cfg = W.search()
    v, q, seg = cfg["values"], cfg["queries"], cfg["segments"]
    gu.say("search full size")
    out, val = sr.galloping_search(gu.to_gpu(v), gu.to_gpu(q), gu.to_gpu(seg),
                                   max_query_count=cfg["max_query_count"], queries_per_tile=cfg["queries_per_tile"])
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert int(val.cpu().view(torch.int32).item()) == 0
    qseg = np.repeat(np.arange(seg.shape[0]), seg[:, 3])
    vo, vc = seg[qseg, 0], seg[qseg, 1]
    assert ((out >= vo) & (out <= vo + vc)).all()
    below = out > vo
    assert (v[out[below] - 1] < q[below]).all()
    inside = out < vo + vc
    assert (v[out[inside]] >= q[inside]).all()
    rng = np.random.default_rng(0)
    for s in rng.choice(seg.shape[0], 96, replace=False):
        a, n, b, m = seg[s]
        sub = np.array([[0, n, 0, m]])
        want, word = oracle.lower_bounds(v[a:a + n], q[b:b + m], sub, max_qc=cfg["max_query_count"],
                                         tile=cfg["queries_per_tile"])
        assert word == 0 and np.array_equal(out[b:b + m] - a, want), s


def test_tile_extremes_in_the_staged_kernel():
    """One query per tile (T = 1): a query below the previous one is in a new
    tile, so no bit 4; one tile for the whole record (T >= qc): it is bit 4.
    Both with a record count small enough for the per-record kernel
    (max_query_count / T <= 256)."""
    rng = np.random.default_rng(41)
    v = np.sort(rng.standard_normal(3000)).astype(np.float32)
    q = np.sort(rng.standard_normal(200))[::-1].astype(np.float32).copy()  # decreasing
    seg = np.array([[0, 3000, 0, 100], [500, 2000, 100, 100]])
    _check(v, q, seg, what="T=1, decreasing", tile=1, max_qc=200)
    _check(v, q, seg, what="T=qc, decreasing", tile=100)
    _check(v, q, seg, what="T>qc, decreasing", tile=100_000)
    qs = q.copy()
    qs[37] = np.nan
    _check(v, qs, seg, what="T=7 with a NaN", tile=7)
