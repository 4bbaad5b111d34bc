"""Parity of the HIP scatter path (segred_scatter_reduce,
segred_offsets_from_index) with the CPU oracle (GPU only).

Bars:
  - integer sums, min/max values and their rows, offsets: bit for bit;
  - float32 sums: the scatter path adds with float32 atomics in arrival order,
    so the bound is the one for n - 1 float32 additions in any order
    (recursive summation, any order and any tree):
    |gpu - ref| <= gamma(n - 1) * sum|x|, gamma(k) = k u / (1 - k u),
    u = 2^-24, for an output reached by n rows (0 for n <= 1: one addition
    to +0.0 is exact); for n <= 160 this is tighter than 1e-5 * sum|x|;
  - float32 means: that bound / n plus one rounding of the quotient.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = 2.0 ** -24


def _gamma(k):
    k = np.asarray(k, dtype=np.float64)
    return np.where(k > 0, k * U / (1 - k * U), 0.0)


def _counts(index, dim):
    inr = (index >= 0) & (index < dim)
    return np.bincount(index[inr], minlength=dim).astype(np.int64) if dim else np.zeros(0, np.int64)


def _run(values_np, index_np, dim, op, want_arg=True, values_t=None, index_t=None):
    import segmented_reduction_amd as sr
    v = values_t if values_t is not None else gu.to_gpu(values_np)
    i = index_t if index_t is not None else gu.to_gpu(index_np)
    out, arg = sr.scatter(v, i, dim, op, want_arg=want_arg)
    torch.cuda.synchronize()
    out_np = out.cpu().numpy().reshape(dim, -1)
    arg_np = arg.cpu().numpy().reshape(dim, -1) if arg is not None else None
    return out_np, arg_np


def _assert_scatter(values_np, index_np, dim, op, out_np, arg_np, orc=None, what=""):
    kind = gu.kind_of(values_np)
    orc = orc or oracle.scatter(values_np, index_np, dim, op)
    assert out_np.shape == orc.out.shape, (what, out_np.shape, orc.out.shape)
    if op in ("min", "max") or kind != "f32":
        ob, rb = out_np.view(np.uint32), orc.out.view(np.uint32)
        if not np.array_equal(ob, rb):
            bad = np.argwhere(ob != rb)[:5]
            raise AssertionError(f"{what} {kind} {op}: values differ at {bad.tolist()}: "
                                 f"gpu {[int(ob[tuple(b)]) for b in bad]} oracle {[int(rb[tuple(b)]) for b in bad]}")
        if arg_np is not None and not np.array_equal(arg_np, orc.arg):
            bad = np.argwhere(arg_np != orc.arg)[:5]
            raise AssertionError(f"{what} {kind} {op}: rows differ at {bad.tolist()}: "
                                 f"gpu {[int(arg_np[tuple(b)]) for b in bad]} "
                                 f"oracle {[int(orc.arg[tuple(b)]) for b in bad]}")
        return orc
    n = _counts(index_np, dim).reshape(dim, 1)
    diff = np.abs(out_np.astype(np.float64) - orc.ref)
    tol = _gamma(n - 1) * orc.mag * 1.0001 + 1e-30
    if op == "mean":
        tol = tol / np.maximum(n, 1) + 1.0001 * U * np.abs(orc.ref) + 1e-30
        assert (out_np[n[:, 0] == 0] == 0).all() and not np.signbit(out_np[n[:, 0] == 0]).any(), what
    if not (diff <= tol).all():
        bad = np.argwhere(diff > tol)[:5]
        raise AssertionError(f"{what} f32 {op}: |gpu-ref| > tol at {bad.tolist()}: "
                             f"diff {[float(diff[tuple(b)]) for b in bad]} tol {[float(tol[tuple(b)]) for b in bad]}")
    return orc


def _check(index_np, values_np, dim, op, what="", want_arg=True):
    gu.say(f"scatter {what} op={op} dtype={gu.kind_of(values_np)} shape={values_np.shape} dim={dim}")
    out_np, arg_np = _run(values_np, index_np, dim, op, want_arg=want_arg)
    return _assert_scatter(values_np, index_np, dim, op, out_np, arg_np if want_arg else None, what=what)


def _ops(kind):
    return ("sum", "min", "max", "mean") if kind == "f32" else ("sum", "min", "max")


# ---------------------------------------------------------------- printed example

@pytest.mark.parametrize("kind", ["u32", "i32", "f32"])
def test_worked_example_as_index(kind):
    """luma.gl GPUSegmentedReduction, 'What is segmented reduction?', with the
    segments written as a destination index, in order and shuffled."""
    with open(os.path.join(GOLDEN, "segmented_reduction_worked_example.json")) as fh:
        g = json.load(fh)
    off = np.array(g["offsets"], dtype=np.int64)
    idx = np.repeat(np.arange(len(off) - 1), np.diff(off)).astype(np.int64)
    vals = np.array(g["values"], dtype={"u32": np.uint32, "i32": np.int32, "f32": np.float32}[kind])
    perm = np.random.default_rng(1).permutation(len(idx))
    for op in ("sum", "min", "max"):
        gu.say(f"scatter worked example {kind} {op}")
        out, arg = _run(vals, idx, 3, op)
        assert out[:, 0].tolist() == g[op]
        if op != "sum":
            assert arg[:, 0].tolist() == g["derived"]["arg" + op]
        out, arg = _run(vals[perm], idx[perm], 3, op)
        assert out[:, 0].tolist() == g[op]
        if op != "sum":
            assert perm[arg[:, 0]].tolist() == g["derived"]["arg" + op]


# ---------------------------------------------------------------- seeded parity grid

CASES = [
    # (seed, rows, dim, feat, order, out_of_range)
    (1, 20_000, 300, 1, "random", 0.0),
    (2, 20_000, 300, 1, "sorted", 0.05),
    (3, 20_000, 5_000, 1, "runs", 0.02),
    (4, 3_000, 1, 1, "one", 0.0),
    (5, 7_777, 130, 2, "random", 0.03),
    (6, 7_777, 130, 3, "runs", 0.0),
    (7, 5_000, 64, 5, "sorted", 0.0),
    (8, 4_000, 250, 16, "random", 0.1),
    (9, 3_001, 90, 64, "random", 0.0),
    (10, 3_001, 90, 64, "runs", 0.05),
    (11, 1_500, 40, 65, "random", 0.0),
    (12, 1_500, 40, 100, "sorted", 0.02),
    (13, 1_000, 33, 130, "random", 0.0),
    (14, 1_000, 33, 200, "runs", 0.0),
    (15, 129, 1_000, 7, "random", 0.0),  # most outputs empty
]


@pytest.mark.parametrize("kind", ["f32", "i32", "u32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"r{c[1]}-d{c[2]}-f{c[3]}-{c[4]}")
def test_scatter_parity(case, kind):
    seed, rows, dim, feat, order, oor = case
    index, vals = W.scatter_case(seed, rows, dim, feat=feat, dtype=kind, order=order, out_of_range=oor)
    for op in _ops(kind):
        _check(index, vals, dim, op, what=f"seed={seed} {order}")
    # ties: the lowest row must win
    index, vals = W.scatter_case(seed + 100, rows, dim, feat=feat, dtype=kind, order=order, out_of_range=oor,
                                 values="ties")
    for op in ("min", "max"):
        _check(index, vals, dim, op, what=f"ties seed={seed} {order}")


@pytest.mark.parametrize("feat", [1, 8, 70])
def test_scatter_without_arg(feat):
    """MIN/MAX without arg_out keep the packed words in library scratch."""
    index, vals = W.scatter_case(21, 9_000, 700, feat=feat, dtype="i32", order="random", values="ties")
    for op in ("min", "max"):
        _check(index, vals, 700, op, what="no arg", want_arg=False)


def test_scatter_degenerate_inputs():
    import segmented_reduction_amd as sr
    # no rows: every output empty
    for kind, dt in (("f32", np.float32), ("i32", np.int32)):
        vals = np.zeros((0, 3), dtype=dt)
        idx = np.zeros(0, dtype=np.int64)
        for op in _ops(kind):
            gu.say(f"scatter no rows {kind} {op}")
            out, arg = _run(vals, idx, 5, op)
            assert (out == 0).all() and not np.signbit(out.astype(np.float32)).any()
            if arg is not None:
                assert (arg == -1).all()
    # no outputs: nothing written, no error
    gu.say("scatter dim_size 0")
    out, arg = sr.scatter(gu.to_gpu(np.ones((10, 2), np.float32)), gu.to_gpu(np.arange(10)), 0, "max")
    torch.cuda.synchronize()
    assert out.shape == (0, 2) and arg.shape == (0, 2)
    # every index out of range
    idx = np.array([-1, 5, 2 ** 40, -(2 ** 62)] * 50, dtype=np.int64)
    vals = np.arange(200, dtype=np.float32)
    for op in ("sum", "min", "max", "mean"):
        _check(idx, vals, 5, op, what="all out of range")
    # one row, one output; -0.0 sums to +0.0 like the oracle's float64 sum
    _check(np.array([0], np.int64), np.array([-0.0], np.float32), 1, "sum", what="negative zero")
    for op in ("sum", "min", "max", "mean"):
        _check(np.array([0], np.int64), np.array([3.5], np.float32), 1, op, what="single row")


def test_scatter_repeatability():
    """Integer sums and min/max with rows repeat bit for bit; float sums stay
    inside the bound on every run (their last bits may move)."""
    index, vals = W.scatter_case(31, 60_000, 100, feat=4, dtype="i32", order="random")
    vf = vals.astype(np.float32) * np.float32(1e-6)
    first = {}
    for rep in range(3):
        for op in ("sum", "min", "max"):
            gu.say(f"scatter repeat {rep} {op}")
            out, arg = _run(vals, index, 100, op)
            if rep == 0:
                first[op] = (out.copy(), None if arg is None else arg.copy())
                _assert_scatter(vals, index, 100, op, out, arg)
            else:
                assert np.array_equal(out, first[op][0]), op
                if arg is not None:
                    assert np.array_equal(arg, first[op][1]), op
        _check(index, vf, 100, "sum", what=f"float repeat {rep}")


# ---------------------------------------------------------------- few outputs (private LDS copies)

PRIVATE = [
    # (seed, rows, dim, feat, order, out_of_range): many elements per output cell
    (51, 120_000, 1, 1, "random", 0.0),
    (52, 150_000, 100, 1, "random", 0.1),
    (53, 200_000, 7, 3, "runs", 0.02),
    (54, 110_000, 100, 8, "random", 0.0),
    (55, 105_000, 60, 16, "sorted", 0.05),
    (56, 70_000, 3, 100, "random", 0.0),
    # >= 128 elements per cell, at least one workgroup per CU
    (57, 200_000, 1000, 1, "sorted", 0.0),
    (58, 300_000, 1000, 4, "random", 0.05),
    (59, 600_000, 500, 8, "runs", 0.0),  # float sums: global atomics (no per-wave copies); others private
    # just eligible, a grid of one or a few workgroups (no first fold stage)
    (61, 200, 1, 1, "random", 0.0),
    (62, 1_200, 2, 3, "sorted", 0.1),
    (63, 3_000, 1, 9, "random", 0.0),
]


@pytest.mark.parametrize("kind", ["f32", "i32", "u32"])
@pytest.mark.parametrize("case", PRIVATE, ids=lambda c: f"r{c[1]}-d{c[2]}-f{c[3]}-{c[4]}")
def test_scatter_few_outputs(case, kind):
    """Many rows into few outputs: each workgroup reduces into a private copy
    in LDS (one copy per wave for float sums of >= 8 features), stores it to
    its own scratch slot, and a fold kernel combines the copies."""
    seed, rows, dim, feat, order, oor = case
    index, vals = W.scatter_case(seed, rows, dim, feat=feat, dtype=kind, order=order, out_of_range=oor,
                                 values="ties" if kind != "f32" else "normal")
    for op in _ops(kind):
        _check(index, vals, dim, op, what=f"few outputs seed={seed}")


@pytest.mark.parametrize("feat", [8, 16, 100])
def test_scatter_few_outputs_float_sums_repeat(feat):
    """Float sums into few outputs with >= 8 features add in a fixed order
    (per-wave copies, then the copies in wave and workgroup order): two calls
    give the same bits, for sum and mean."""
    index, vals = W.scatter_case(60 + feat, 200_000, 16, feat=feat, dtype="f32", order="random", out_of_range=0.01)
    for op in ("sum", "mean"):
        gu.say(f"scatter few-output repeat F={feat} {op}")
        a, _ = _run(vals, index, 16, op, want_arg=False)
        b, _ = _run(vals, index, 16, op, want_arg=False)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        _assert_scatter(vals, index, 16, op, a, None, what=f"few-output repeat F={feat}")


# ---------------------------------------------------------------- index -> offsets

OFFSET_CASES = [
    # (seed, rows, dim, order, out_of_range)
    (1, 0, 0, "random", 0.0),
    (2, 0, 10, "random", 0.0),
    (3, 10, 0, "random", 0.0),
    (4, 1, 1, "one", 0.0),
    (5, 50_000, 4095, "sorted", 0.0),
    (6, 50_000, 4096, "random", 0.1),
    (7, 50_000, 4097, "runs", 0.02),
    (8, 200_000, 10_000, "sorted", 0.0),
    (9, 100_000, 300_000, "random", 0.05),
    (10, 70_000, 3, "one", 0.01),
    (11, 1_000_001, 20_000, "runs", 0.0),
]


@pytest.mark.parametrize("case", OFFSET_CASES, ids=lambda c: f"r{c[1]}-d{c[2]}-{c[3]}")
def test_offsets_from_index_parity(case):
    import segmented_reduction_amd as sr
    seed, rows, dim, order, oor = case
    index, _ = W.scatter_case(seed, rows, dim, feat=1, order=order, out_of_range=oor)
    gu.say(f"offsets_from_index rows={rows} dim={dim} {order} oor={oor}")
    got = sr.offsets_from_index(gu.to_gpu(index), dim)
    torch.cuda.synchronize()
    want = oracle.offsets_from_index(index, dim)
    assert np.array_equal(got.cpu().numpy(), want)


def test_index_offsets_feed_the_segmented_reduction():
    """graph-reduce README, 'Usage': a destination-sorted index -> CSR pointer
    -> segment reduction without atomics; equals the scatter of the same rows
    (exact for integers, min/max and rows)."""
    import segmented_reduction_amd as sr
    index, vals = W.scatter_case(41, 120_000, 3_000, feat=8, dtype="i32", order="sorted")
    gu.say("index -> offsets -> reduce")
    it, vt = gu.to_gpu(index), gu.to_gpu(vals)
    off = sr.offsets_from_index(it, 3_000)
    for op in ("sum", "min", "max"):
        out, arg = sr.reduce(vt, off, op)
        torch.cuda.synchronize()
        orc = oracle.scatter(vals, index, 3_000, op)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), orc.out.view(np.uint32)), op
        if arg is not None:
            assert np.array_equal(arg.cpu().numpy(), orc.arg), op


# ---------------------------------------------------------------- full size

@pytest.mark.parametrize("feat", [64, 16])
def test_scatter_full_size(feat):
    """1,000,000 rows x F float32 into 10,000 outputs, unsorted index (the
    graph-reduce README's measured shape); the whole output is compared."""
    import segmented_reduction_amd as sr
    cfg = W.scatter(feat=feat)
    index, vals, dim = cfg["index"], cfg["f32"], cfg["dim"]
    it, vt = gu.to_gpu(index), gu.to_gpu(vals)
    for op in ("sum", "max", "mean"):
        gu.say(f"scatter full size F={feat} {op}")
        out, arg = _run(vals, index, dim, op, values_t=vt, index_t=it)
        _assert_scatter(vals, index, dim, op, out, arg, what=f"full F={feat}")
    gu.say(f"offsets_from_index full size F={feat}")
    srt = np.sort(index)
    got = sr.offsets_from_index(gu.to_gpu(srt), dim)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.offsets_from_index(srt, dim))


# ---------------------------------------------------------------- exact float sums on every path

# (rows, outputs, features, path the call takes): many outputs -> one global
# atomic per element; few outputs (one copy fits 32 KB, >= 128 elements per
# output cell) -> private LDS copies with LDS atomics (F < 8) or one copy per
# wave with fixed-order adds (float sums of F >= 8).
EXACT_CASES = [
    (400_000, 10_000, 1, "element atomics"),
    (400_000, 10_000, 4, "element atomics"),
    (200_000, 5_000, 16, "element atomics"),
    (300_000, 100, 1, "private copies, LDS atomics"),
    (200_000, 200, 4, "private copies, LDS atomics"),
    (100_000, 100, 16, "private copies, one per wave"),
    (100_000, 8, 64, "private copies, one per wave"),
]


@pytest.mark.parametrize("rows,dim,feat,path", EXACT_CASES)
def test_integer_valued_float_sums_are_exact(rows, dim, feat, path):
    """Float32 values in {-3..3} whose partial sums stay below 2^24 add
    exactly in any order: on every path the scatter sum must equal the
    oracle's bit for bit, so a dropped, doubled or misrouted row fails."""
    rng = np.random.default_rng(rows + dim + feat)
    idx = rng.integers(0, dim, rows, dtype=np.int64)
    shape = (rows,) if feat == 1 else (rows, feat)
    vals = rng.integers(-3, 4, shape).astype(np.float32)
    assert np.bincount(idx, minlength=dim).max() * 3 < 2 ** 24
    gu.say(f"scatter exact sum {path} rows={rows} dim={dim} F={feat}")
    out, _ = _run(vals, idx, dim, "sum")
    orc = oracle.scatter(vals, idx, dim, "sum")
    assert np.array_equal(out.view(np.uint32), orc.out.view(np.uint32)), path
    assert np.array_equal(out.astype(np.float64), orc.ref), path


@pytest.mark.parametrize("rows,dim,feat", [(100_000, 100, 16), (100_000, 8, 64), (60_000, 30, 32)])
def test_fixed_order_float_sums_meet_the_reduction_bar(rows, dim, feat):
    """The per-wave-copy path adds in a fixed order: its float sums meet the
    segmented reduction's bar, 1e-5 * sum|x| + 1e-6 per output, and repeat
    bit for bit."""
    rng = np.random.default_rng(rows + feat)
    idx = rng.integers(0, dim, rows, dtype=np.int64)
    vals = rng.standard_normal((rows, feat), dtype=np.float32)
    gu.say(f"scatter fixed-order sum rows={rows} dim={dim} F={feat}")
    out, _ = _run(vals, idx, dim, "sum")
    orc = oracle.scatter(vals, idx, dim, "sum")
    assert (np.abs(out.astype(np.float64) - orc.ref) <= 1e-5 * orc.mag + 1e-6).all()
    again, _ = _run(vals, idx, dim, "sum")
    assert np.array_equal(out.view(np.uint32), again.view(np.uint32))
