"""Parity of the HIP segmented reduction with the CPU oracle (GPU only).

Every call goes through the C ABI (libsegred.so) via the binding.  Integer
sums, min/max values and rows must match bit for bit; float32 sums within
1e-5 * sum|x| + 1e-6 per (segment, feature) (means: that bound / length).
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
NP_T = {"u32": np.uint32, "i32": np.int32, "f32": np.float32}


@pytest.fixture(autouse=True)
def _reset_shares():
    import segmented_reduction_amd as sr
    sr.set_shares(0)
    yield
    sr.set_shares(0)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


@pytest.mark.parametrize("kind", ["u32", "i32", "f32"])
def test_worked_example(kind):
    """luma.gl GPUSegmentedReduction, 'What is segmented reduction?'."""
    g = _golden("segmented_reduction_worked_example.json")
    vals = np.array(g["values"], dtype=NP_T[kind])
    off = np.array(g["offsets"], dtype=np.int64)
    for op in ("sum", "min", "max"):
        gu.say(f"worked example {kind} {op}")
        out, arg = gu.run_gpu(vals, off, op)
        assert out[:, 0].tolist() == g[op]
        if op != "sum":
            assert arg[:, 0].tolist() == g["derived"]["arg" + op]


@pytest.mark.parametrize("kind", ["u32", "i32", "f32"])
def test_empty_segments_fixture(kind):
    g = _golden("empty_segments.json")
    vals = np.array(g["values"], dtype=NP_T[kind])
    off = np.array(g["offsets"], dtype=np.int64)
    for op in ("sum", "min", "max"):
        gu.say(f"empty fixture {kind} {op}")
        out, arg = gu.run_gpu(vals, off, op)
        assert out[:, 0].tolist() == g[op]
        if op != "sum":
            assert arg[:, 0].tolist() == g["arg" + op]


FEATS = [1, 2, 3, 4, 5, 6, 8, 12, 16, 24, 32, 33, 64, 65, 128, 256, 260]


@pytest.mark.parametrize("feat", FEATS)
@pytest.mark.parametrize("kind", ["u32", "i32", "f32"])
def test_random_ragged(kind, feat):
    """Ragged segments, 10 % empty, one long segment, offsets[0] > 0, unread
    rows after the last offset; several work partitions (share counts)."""
    rows_target = 60_000 if feat <= 8 else 6_000
    mean_len = 12
    segs = max(4, rows_target // (mean_len + 1))
    off, vals = W.ragged(seed=feat * 7 + len(kind), segments=segs, mean_len=mean_len, feat=feat, dtype=kind,
                         empty_frac=0.1, base=5, tail_rows=3, long_segment=rows_target // 3)
    ops = ["sum", "min", "max"] + (["mean"] if kind == "f32" else [])
    for op in ops:
        orc = oracle.reduce(vals, off, op)
        for shares in (None, 1, 3, 64, 997):
            gu.say(f"ragged kind={kind} F={feat} op={op} shares={shares} S={segs}")
            out, arg = gu.run_gpu(vals, off, op, shares=shares)
            gu.assert_parity(vals, off, op, out, arg, orc=orc, what=f"ragged F={feat} shares={shares}")


@pytest.mark.parametrize("feat", [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 64])
@pytest.mark.parametrize("kind", ["u32", "i32", "f32"])
def test_ties_go_to_lower_row(kind, feat):
    off, vals = W.ragged(seed=100 + feat, segments=2000, mean_len=15, feat=feat, dtype=kind, values="ties",
                         long_segment=5000)
    for op in ("min", "max"):
        for shares in (None, 7, 333):
            out, arg = gu.run_gpu(vals, off, op, shares=shares)
            gu.assert_parity(vals, off, op, out, arg, what=f"ties F={feat} shares={shares}")


@pytest.mark.parametrize("feat", [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 64, 5])
def test_integer_valued_floats_sum_exactly(feat):
    """Small integer-valued floats add exactly in any order: the GPU sum must
    equal the oracle's bit for bit (pins indexing independently of rounding)."""
    off, vals = W.ragged(seed=200 + feat, segments=3000, mean_len=20, feat=feat, values="intfloat",
                         long_segment=20000, base=2)
    for shares in (None, 5, 1024):
        gu.say(f"intfloat F={feat} shares={shares}")
        out, _ = gu.run_gpu(vals, off, "sum", shares=shares)
        orc = oracle.reduce(vals, off, "sum")
        assert np.array_equal(out.view(np.uint32), orc.out.view(np.uint32))


def test_repeat_runs_are_bitwise_identical():
    off, vals = W.ragged(seed=5, segments=20000, mean_len=40, feat=1, long_segment=300000)
    v, o = gu.to_gpu(vals), gu.to_gpu(off)
    import segmented_reduction_amd as sr
    first = None
    for rep in range(5):
        gu.say(f"determinism rep {rep}")
        out, _ = sr.reduce(v, o, "sum")
        b = out.cpu().numpy().tobytes()
        first = first or b
        assert b == first


def test_single_segment_is_a_global_reduction():
    rng = np.random.default_rng(1)
    vals = rng.standard_normal(3_000_000).astype(np.float32)
    off = np.array([123, 2_999_000], dtype=np.int64)
    for op in ("sum", "min", "max", "mean"):
        gu.check(vals, off, op, what="S=1")
    ints = rng.integers(-10, 10, 3_000_000, dtype=np.int32)
    for op in ("min", "max"):
        out, arg = gu.run_gpu(ints, off, op)
        seg = ints[123:2_999_000]
        want = seg.min() if op == "min" else seg.max()
        first = 123 + int(np.flatnonzero(seg == want)[0])
        assert out[0, 0] == want and arg[0, 0] == first


def test_all_segments_empty():
    off = np.full(5001, 7, dtype=np.int64)
    for kind in ("u32", "i32", "f32"):
        vals = np.ones((10, 4), dtype=NP_T[kind])
        for op in ("sum", "min", "max") + (("mean",) if kind == "f32" else ()):
            out, arg = gu.run_gpu(vals, off, op)
            assert (out == 0).all()
            if arg is not None:
                assert (arg == -1).all()


def test_every_segment_one_row():
    vals = np.arange(100_000, dtype=np.int32)[::-1].copy()
    off = np.arange(100_001, dtype=np.int64)
    for op in ("sum", "min", "max"):
        out, arg = gu.run_gpu(vals, off, op)
        assert np.array_equal(out[:, 0], vals)
        if arg is not None:
            assert np.array_equal(arg[:, 0], np.arange(100_000))


def test_zero_segments_is_a_no_op():
    import segmented_reduction_amd as sr
    v = torch.ones(10, device="cuda")
    o = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, arg = sr.reduce(v, o, "max")
    torch.cuda.synchronize()
    assert out.shape == (0,) and arg.shape == (0,)


@pytest.mark.parametrize("feat", [3, 4, 6, 24, 31, 32])
def test_unaligned_rows_use_the_scalar_path(feat):
    """values starting 4 bytes past an allocation: 16- and 8-byte pieces per
    lane do not apply and the 4-byte path must give the same results (rows
    of 3 features also load 16-byte units from a 4-byte aligned chunk)."""
    off, vals = W.ragged(seed=9 + feat, segments=3000, mean_len=10, feat=feat, dtype="f32")
    big = torch.zeros(vals.size + 1, dtype=torch.float32, device="cuda")
    big[1:] = gu.to_gpu(vals.reshape(-1))
    v = big[1:].view(vals.shape)
    assert v.data_ptr() % 16 != 0
    for op in ("sum", "max"):
        out, arg = gu.run_gpu(vals, off, op, values_t=v)
        gu.assert_parity(vals, off, op, out, arg, what="unaligned")


def test_value_only_min_max():
    off, vals = W.ragged(seed=10, segments=500, mean_len=30, feat=32, dtype="i32")
    for op in ("min", "max"):
        out, arg = gu.run_gpu(vals, off, op, want_arg=False)
        assert arg is None
        gu.assert_parity(vals, off, op, out, None, what="value-only")


def test_guard_bands_are_untouched():
    """Outputs written into the middle of larger buffers: the bytes around
    them keep their canary values."""
    import segmented_reduction_amd as sr
    off, vals = W.ragged(seed=11, segments=777, mean_len=9, feat=8, dtype="u32")
    s = off.size - 1
    pad = 64
    out_big = torch.full((s * 8 + 2 * pad,), -1515870811, dtype=torch.int32, device="cuda")
    arg_big = torch.full((s * 8 + 2 * pad,), -12345, dtype=torch.int64, device="cuda")
    out_view = out_big[pad:pad + s * 8].view(torch.uint32).view(s, 8)
    arg_view = arg_big[pad:pad + s * 8].view(s, 8)
    sr.reduce(gu.to_gpu(vals), gu.to_gpu(off), "max", out=out_view, arg=arg_view)
    torch.cuda.synchronize()
    ob, ab = out_big.cpu().numpy(), arg_big.cpu().numpy()
    assert (ob[:pad] == np.int32(-1515870811)).all() and (ob[-pad:] == np.int32(-1515870811)).all()
    assert (ab[:pad] == -12345).all() and (ab[-pad:] == -12345).all()
    gu.assert_parity(vals, off, "max", out_view.cpu().numpy().reshape(s, 8), arg_view.cpu().numpy(), what="guard")


def test_three_dimensional_values_flatten_features():
    off, vals = W.ragged(seed=12, segments=400, mean_len=7, feat=12, dtype="f32")
    v3 = vals.reshape(-1, 3, 4)
    import segmented_reduction_amd as sr
    out, arg = sr.reduce(gu.to_gpu(v3), gu.to_gpu(off), "min")
    assert out.shape == (400, 3, 4) and arg.shape == (400, 3, 4)
    gu.assert_parity(vals, off, "min", out.cpu().numpy().reshape(400, 12), arg.cpu().numpy().reshape(400, 12))


def _edge_offsets(chunk=2048):
    """1-D lengths that put segment ends on chunk edges for a single share
    starting at row 0: ends exactly at multiples of the chunk, runs of 300
    empty segments inside a chunk and on a chunk edge, a segment spanning
    several chunks, stretches with more ends than one chunk takes, and a
    last segment ending inside a partial chunk."""
    lengths = [chunk, chunk, 5, chunk - 5, 2 * chunk, 1, chunk - 1]
    lengths += [0] * 300 + [7, 100] + [0] * 300 + [chunk - 107]
    lengths += [3 * chunk + 17, chunk - 17] + [0] * 5 + [11, 0, 0, 29]
    # more ends than one chunk holds: 700 empty segments at one position,
    # then 1500 one-row segments and 600 two-row ones
    lengths += [0] * 700 + [1] * 1500 + [2] * 600 + [chunk // 2]
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


@pytest.mark.parametrize("kind", ["u32", "i32", "f32"])
def test_one_dimensional_chunk_edges(kind):
    off = _edge_offsets()
    rows = int(off[-1])
    rng = np.random.default_rng(77)
    vals = {"f32": rng.standard_normal(rows, dtype=np.float32),
            "i32": rng.integers(-(2 ** 31), 2 ** 31, rows, dtype=np.int32),
            "u32": rng.integers(0, 2 ** 32, rows, dtype=np.uint32)}[kind]
    ops = ["sum", "min", "max"] + (["mean"] if kind == "f32" else [])
    for op in ops:
        orc = oracle.reduce(vals, off, op)
        for shares in (1, 2, 3, None):
            gu.say(f"chunk edges kind={kind} op={op} shares={shares}")
            out, arg = gu.run_gpu(vals, off, op, shares=shares)
            gu.assert_parity(vals, off, op, out, arg, orc=orc, what=f"chunk edges shares={shares}")


@pytest.mark.parametrize("kind", ["i32", "f32"])
def test_one_dimensional_weighted_shares(kind):
    """The 1-D kernel weighs a segment end as 8 rows in its shares: share
    boundaries then fall inside long stretches of empty segments (each is 8
    items with no rows), inside stretches of one-row segments and inside long
    segments, and each must stop at a point of the merged sequence.  Many
    share counts move the boundaries across all three."""
    rng = np.random.default_rng(91)
    lengths = np.concatenate([
        [50_000], np.zeros(40_000, np.int64), [3], np.ones(30_000, np.int64), np.zeros(7, np.int64),
        rng.integers(0, 4, 20_000), [120_000], np.zeros(25_000, np.int64), rng.integers(1, 60, 2_000)])
    off = np.concatenate([[5], 5 + np.cumsum(lengths)]).astype(np.int64)  # offsets[0] > 0
    rows = int(off[-1])
    vals = {"f32": rng.standard_normal(rows, dtype=np.float32),
            "i32": rng.integers(-1000, 1000, rows, dtype=np.int32)}[kind]
    for op in ("sum", "min", "max"):
        orc = oracle.reduce(vals, off, op)
        for shares in (None, 4, 36, 412, 4096):
            gu.say(f"weighted shares kind={kind} op={op} shares={shares}")
            out, arg = gu.run_gpu(vals, off, op, shares=shares)
            gu.assert_parity(vals, off, op, out, arg, orc=orc, what=f"weighted shares={shares}")


@pytest.mark.parametrize("feat", [1, 32, 65, 100, 260])
@pytest.mark.parametrize("kind", ["u32", "f32"])
def test_values_end_with_their_buffer(kind, feat):
    """No unread rows after the last offset, and the values view ends exactly
    at the end of its tensor's storage (a multiple of 2 MiB, so the caching
    allocator has no slack to hide a read past it): every kernel's last
    chunk or part must stop at offsets[S]."""
    off, vals = W.ragged(seed=300 + feat, segments=1500, mean_len=9, feat=feat, dtype=kind, empty_frac=0.1,
                         base=0, tail_rows=0, long_segment=2000)
    rows = int(off[-1])
    elems = rows * feat
    total = -(-(elems * 4) // (2 << 20)) * (2 << 20) // 4
    import segmented_reduction_amd as sr
    torch_dt = {"u32": torch.int32, "f32": torch.float32}[kind]
    buf = torch.empty(total, dtype=torch_dt, device="cuda")
    view = buf[total - elems:]
    view.copy_(torch.from_numpy(vals.reshape(-1).view(np.int32 if kind == "u32" else np.float32)).cuda())
    v = view.view(torch.uint32 if kind == "u32" else torch.float32).reshape((rows,) if feat == 1 else (rows, feat))
    o = gu.to_gpu(off)
    for op in ("sum", "max") + (("mean",) if kind == "f32" else ()):
        for shares in (None, 3, 64):
            gu.say(f"end-of-buffer kind={kind} F={feat} op={op} shares={shares}")
            if shares:
                sr.set_shares(shares)
            try:
                out, arg = sr.reduce(v, o, op)
                torch.cuda.synchronize()
            finally:
                sr.set_shares(0)
            s = len(off) - 1
            gu.assert_parity(vals, off, op, out.cpu().numpy().reshape(s, -1),
                             arg.cpu().numpy().reshape(s, -1) if arg is not None else None,
                             what=f"end-of-buffer F={feat} shares={shares}")


@pytest.mark.parametrize("dtype,op,feat", [(2, 0, 1), (2, 1, 1), (0, 0, 1), (1, 2, 1), (2, 0, 32), (2, 2, 32),
                                           (2, 3, 32), (2, 0, 64), (2, 2, 64), (2, 0, 8), (0, 1, 3), (2, 2, 100),
                                           (2, 2, 260)])
def test_default_shares_fit_one_round(dtype, op, feat):
    """The share count is a constant of each kernel (the same on every
    device); on MI355X it must not exceed the waves that fit at once, so a
    call runs as one round of waves."""
    import segmented_reduction_amd as sr
    lib = sr.library()
    shares = lib.segred_get_shares(dtype, op, feat)
    resident = lib.segred_resident_waves(dtype, op, feat)
    assert 0 < shares <= resident, (shares, resident)


# Bit patterns at the ends of each type's order (graph-reduce README,
# "Method": the order key; luma.gl GPUSegmentedReduction, "Contract": an
# empty segment gives the identity and -1).  Max over the lowest key and min
# over the highest are the cases where every element equals the identity's
# key: the result must still be the segment's first row, and an empty
# segment must still give -1.
_LOWEST = {"u32": 0x00000000, "i32": 0x80000000, "f32": 0xFFFFFFFF}   # order key 0
_HIGHEST = {"u32": 0xFFFFFFFF, "i32": 0x7FFFFFFF, "f32": 0x7FFFFFFF}  # order key 0xFFFFFFFF


@pytest.mark.parametrize("feat", [1, 3, 4, 8, 32, 64, 100])
@pytest.mark.parametrize("kind", ["u32", "i32", "f32"])
def test_extreme_keys_keep_the_first_row(kind, feat):
    rng = np.random.default_rng(7000 + feat)
    off, _ = W.ragged(seed=7100 + feat, segments=1500, mean_len=12, feat=feat, dtype=kind, long_segment=3000)
    rows = int(off[-1])
    shape = (rows,) if feat == 1 else (rows, feat)
    for op, pat in (("max", _LOWEST[kind]), ("min", _HIGHEST[kind])):
        bits = np.full(shape, pat, dtype=np.uint32)
        for mixed in (False, True):
            b = bits.copy()
            if mixed:
                # a few ordinary values, so positions other than the first win
                # in some segments and rows of equal extreme keys in others
                pick = rng.random(shape) < 0.05
                b[pick] = rng.integers(1, 1 << 30, int(pick.sum()), dtype=np.uint32) | (1 << 30)
            vals = b.view(NP_T[kind])
            for shares in (None, 5, 411):
                gu.say(f"extreme keys kind={kind} F={feat} op={op} mixed={mixed} shares={shares}")
                out, arg = gu.run_gpu(vals, off, op, shares=shares)
                gu.assert_parity(vals, off, op, out, arg, what=f"extreme {kind} F={feat} {op} mixed={mixed}")


@pytest.mark.parametrize("shares,size", [(1, 1024), (2, 1000), (2, 1016), (2, 1024), (3, 1032), (3, 1048), (7, 1028),
                                         (7, 1536), (5, 2040)])
def test_team_share_sizes_near_64k_multiples(shares, size):
    """Rows of 32 features with share sizes (rows + segment ends) within 32
    of a multiple of 512 (64 KB of rows): the kernel grows the share size to
    the band's edge, so the last shares are shorter or empty; results must
    not change.  A few long segments, an empty one, a unit one."""
    rng = np.random.default_rng(shares * 10007 + size)
    segs = 6
    total = shares * size - segs  # items = rows + segment ends
    cuts = np.sort(rng.integers(0, total - 1, segs - 3))
    lens = np.diff(np.concatenate([[0], cuts, [total - 1]])).astype(np.int64)
    lens = np.concatenate([lens[:1], [0, 1], lens[1:]])
    off = np.zeros(segs + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    assert off[-1] + segs == shares * size and (lens >= 0).all()
    vals = rng.standard_normal((int(off[-1]), 32)).astype(np.float32)
    for op in ("sum", "max", "mean"):
        gu.say(f"team band shares={shares} size={size} op={op}")
        out, arg = gu.run_gpu(vals, off, op, shares=shares)
        gu.assert_parity(vals, off, op, out, arg, what=f"team band shares={shares} size={size}")
