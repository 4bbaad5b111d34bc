"""Parity of the HIP segmented scan (segred_scan) with the CPU oracle (GPU
only).

Bars: integer sums and min/max bit for bit; float32 sums within
2^-24 * |ref| + 2^-30 * sum|x| of the float64 oracle prefix (the kernel
accumulates in float64 and rounds each output once, so the only error
beyond one rounding is float64 reassociation, far below 2^-30 * sum|x|).
Rows outside the segments must keep what the output held before.
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
SENTINEL = 0x5EC7AB1E


@pytest.fixture(autouse=True)
def _reset_shares():
    import segmented_reduction_amd as sr
    sr.set_shares(0)
    yield
    sr.set_shares(0)


def _gpu_scan(vals, off, op, exclusive, shares=None, vals_t=None, off_t=None):
    import segmented_reduction_amd as sr
    v = vals_t if vals_t is not None else gu.to_gpu(vals)
    o = off_t if off_t is not None else gu.to_gpu(off)
    out = torch.full(v.shape, SENTINEL, dtype=torch.int32, device=v.device).view(v.dtype)
    if shares is not None:
        sr.set_shares(shares)
    try:
        sr.scan(v, o, op, exclusive=exclusive, out=out)
        torch.cuda.synchronize()
    finally:
        if shares is not None:
            sr.set_shares(0)
    return out.cpu().numpy().reshape(vals.shape[0], -1)


def _assert_scan(vals, off, op, exclusive, got, what=""):
    kind = gu.kind_of(vals)
    orc = oracle.scan(vals, off, op, exclusive)
    rows = vals.shape[0]
    inside = np.zeros(rows, dtype=bool)
    inside[int(off[0]):int(off[-1])] = True
    gb = got.view(np.uint32)
    assert (gb[~inside] == np.uint32(SENTINEL)).all(), f"{what}: rows outside the segments were written"
    if op != "sum" or kind != "f32":
        rb = orc.out.view(np.uint32)
        if not np.array_equal(gb[inside], rb[inside]):
            bad = np.argwhere(gb != rb)[:5]
            raise AssertionError(f"{what} {kind} {op} excl={exclusive}: differ at {bad.tolist()}: "
                                 f"gpu {[int(gb[tuple(b)]) for b in bad]} oracle {[int(rb[tuple(b)]) for b in bad]}")
        return
    diff = np.abs(got[inside].astype(np.float64) - orc.ref[inside])
    tol = 2.0 ** -24 * np.abs(orc.ref[inside]) * 1.0001 + 2.0 ** -30 * orc.mag[inside] + 1e-30
    if not (diff <= tol).all():
        bad = np.argwhere(diff > tol)[:5]
        raise AssertionError(f"{what} f32 sum excl={exclusive}: |gpu-ref| > tol at {bad.tolist()}: "
                             f"diff {[float(diff[tuple(b)]) for b in bad]} tol {[float(tol[tuple(b)]) for b in bad]}")


def _check(vals, off, op, exclusive, shares=None, what=""):
    gu.say(f"scan {what} op={op} excl={exclusive} dtype={gu.kind_of(vals)} shape={vals.shape} "
           f"S={off.shape[0] - 1} o0={int(off[0])} shares={shares}")
    got = _gpu_scan(vals, off, op, exclusive, shares)
    _assert_scan(vals, off, op, exclusive, got, what)


@pytest.mark.parametrize("kind", ["u32", "i32", "f32"])
def test_printed_reduction_ends(kind):
    """luma.gl GPUSegmentedReduction, 'What is segmented reduction?': the
    inclusive scan ends each segment on the printed result; the exclusive
    scan starts each segment at 0."""
    with open(os.path.join(GOLDEN, "segmented_reduction_worked_example.json")) as fh:
        g = json.load(fh)
    vals = np.array(g["values"], dtype={"u32": np.uint32, "i32": np.int32, "f32": np.float32}[kind])
    off = np.array(g["offsets"], dtype=np.int64)
    for op in ("sum", "min", "max"):
        gu.say(f"scan worked example {kind} {op}")
        inc = _gpu_scan(vals, off, op, False)[:, 0]
        exc = _gpu_scan(vals, off, op, True)[:, 0]
        assert [inc[int(off[s + 1]) - 1] for s in range(3)] == g[op]
        assert all(exc[int(off[s])] == 0 for s in range(3))


CASES = [
    # (seed, segments, mean_len, feat, empty_frac, base, long_segment, tail_rows)
    (1, 300, 40, 1, 0.1, 0, 0, 0),
    (2, 2_000, 5, 1, 0.3, 7, 0, 5),
    (3, 50, 2_000, 1, 0.0, 3, 150_000, 0),
    (4, 700, 30, 2, 0.1, 0, 0, 3),
    (5, 400, 25, 3, 0.2, 11, 0, 0),
    (6, 300, 20, 5, 0.1, 0, 20_000, 0),
    (7, 250, 30, 16, 0.05, 2, 0, 2),
    (8, 200, 20, 32, 0.1, 0, 9_000, 0),
    (9, 120, 15, 33, 0.1, 1, 0, 0),
    (10, 150, 25, 64, 0.1, 0, 5_000, 1),
    (11, 60, 10, 65, 0.2, 0, 0, 0),
    (12, 40, 12, 130, 0.1, 4, 700, 0),
]


@pytest.mark.parametrize("kind", ["f32", "i32", "u32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[1]}-len{c[2]}-f{c[3]}-long{c[6]}")
def test_scan_parity(case, kind):
    seed, segs, mean_len, feat, empty, base, long_seg, tail = case
    off, vals = W.ragged(seed, segs, mean_len, feat=feat, dtype=kind, empty_frac=empty, base=base,
                         long_segment=long_seg, tail_rows=tail)
    for op in ("sum", "min", "max"):
        for exclusive in (False, True):
            _check(vals, off, op, exclusive, what=f"seed={seed}")


@pytest.mark.parametrize("shares", [1, 3, 64, 997])
@pytest.mark.parametrize("feat", [1, 4, 64, 100])
def test_scan_share_counts(shares, feat):
    """Segments cut by many share boundaries, including a long one spread over
    hundreds of shares, and shares that hold no rows."""
    off, vals = W.ragged(40 + feat, 500, 30, feat=feat, dtype="f32", empty_frac=0.3, long_segment=40_000)
    for op, exclusive in (("sum", False), ("max", True), ("min", False)):
        _check(vals, off, op, exclusive, shares=shares, what=f"shares={shares}")
    offi, valsi = W.ragged(50 + feat, 500, 30, feat=feat, dtype="i32", empty_frac=0.3, long_segment=40_000)
    _check(valsi, offi, "sum", True, shares=shares, what=f"int shares={shares}")


def test_scan_degenerate():
    # all segments empty, one row, every segment of one row, S = 0
    off = np.zeros(50, dtype=np.int64) + 3
    _check(np.arange(10, dtype=np.float32), off, "sum", False, what="all empty")
    _check(np.array([2.5], np.float32), np.array([0, 1], np.int64), "sum", True, what="one row")
    _check(np.array([2.5], np.float32), np.array([0, 1], np.int64), "max", False, what="one row")
    off = np.arange(0, 5001, dtype=np.int64)
    vals = np.random.default_rng(3).integers(-5, 5, 5000).astype(np.int32)
    for op in ("sum", "min", "max"):
        _check(vals, off, op, False, what="unit segments")
        _check(vals, off, op, True, what="unit segments")
    import segmented_reduction_amd as sr
    gu.say("scan S = 0")
    out = torch.full((4,), 9, dtype=torch.int32, device="cuda")
    sr.scan(gu.to_gpu(np.arange(4, dtype=np.int32)), gu.to_gpu(np.array([2], np.int64)), "sum", out=out)
    torch.cuda.synchronize()
    assert out.tolist() == [9, 9, 9, 9]


def test_scan_repeats_bitwise():
    off, vals = W.ragged(77, 400, 200, feat=1, dtype="f32", long_segment=300_000)
    gu.say("scan repeat")
    a = _gpu_scan(vals, off, "sum", False)
    for _ in range(2):
        assert np.array_equal(a.view(np.uint32), _gpu_scan(vals, off, "sum", False).view(np.uint32))


@pytest.mark.parametrize("name", ["message", "skew"])
def test_scan_full_size(name):
    """The message-passing (1M x 64 -> 10,000 segments) and heavy-skew (50M
    1-D, one 5M-row segment) inputs at full size, in the bench's launch
    configuration: inclusive sum and exclusive max, every row compared."""
    cfg = getattr(W, name)()
    vals, off = cfg["f32"], cfg["offsets"]
    vt, ot = gu.to_gpu(vals), gu.to_gpu(off)
    for op, exclusive in (("sum", False), ("max", True)):
        gu.say(f"scan full size {name} {op} excl={exclusive}")
        got = _gpu_scan(vals, off, op, exclusive, vals_t=vt, off_t=ot)
        _assert_scan(vals, off, op, exclusive, got, what=f"full {name}")
