"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError on a mismatch.  They are run against the real oracle by
``test_oracle_pins.py`` and against planted mistakes by
``test_oracle_mutants.py`` (every planted mistake must fail at least one pin).

What each pin leans on:
  - printed worked examples (tests/golden/*.json, each with its citation);
  - brute force in pure Python (tests/brute_ref.py) on tiny random inputs;
  - library routines for special cases (numpy reduceat / argmin / argmax,
    itertools.groupby, math.fsum, torch.segment_reduce on the CPU);
  - closed forms (integer wrap-around, integer-valued floats summed exactly);
  - invariants of min/max + arg (gathered back, inside the segment, lowest row
    among ties, nothing better in the segment).
"""
from __future__ import annotations

import itertools
import json
import math
import os
import struct

import numpy as np

import oracle
from tests import brute_ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NP_T = {"u32": np.uint32, "i32": np.int32, "f32": np.float32}


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _col(a):
    return [x[0] for x in a.tolist()]


# ---------------------------------------------------------------- printed examples

def pin_worked_example(lib):
    """luma.gl GPUSegmentedReduction, 'What is segmented reduction?'."""
    g = _golden("segmented_reduction_worked_example.json")
    off = np.array(g["offsets"], dtype=np.int64)
    for kind in ("u32", "i32", "f32"):
        vals = np.array(g["values"], dtype=NP_T[kind])
        for op in ("sum", "min", "max"):
            r = oracle.reduce(vals, off, op, lib=lib)
            assert _col(r.out) == g[op], (kind, op, _col(r.out))
            if op != "sum":
                assert _col(r.arg) == g["derived"]["arg" + op], (kind, op, _col(r.arg))


def pin_empty_segments(lib):
    """Repeated offsets are empty segments; empty -> 0 (arg -1)."""
    g = _golden("empty_segments.json")
    off = np.array(g["offsets"], dtype=np.int64)
    for kind in ("u32", "i32", "f32"):
        vals = np.array(g["values"], dtype=NP_T[kind])
        for op in ("sum", "min", "max"):
            r = oracle.reduce(vals, off, op, lib=lib)
            assert _col(r.out) == g[op], (kind, op)
            if op != "sum":
                assert _col(r.arg) == g["arg" + op], (kind, op)
        if kind == "f32":
            r = oracle.reduce(vals, off, "mean", lib=lib)
            assert _col(r.out) == [0.0, 6.0, 0.0, 1.0, 0.0]
            # zero means all-zero bits (+0.0), not -0.0
            assert not np.signbit(r.out).any()


def pin_rle_examples(lib):
    """luma.gl GPURunLengthEncode, 'What is run-length encoding?' and 'Contract'."""
    g = _golden("run_length_encode_examples.json")
    for case in g["cases"]:
        v, ln, off, c = oracle.rle(np.array(case["input"], dtype=np.uint32), lib=lib)
        assert v.tolist() == case["values"], case["cite"]
        assert c == len(case["values"])
        lengths = case.get("lengths", case.get("derived_lengths"))
        offsets = case.get("offsets", case.get("derived_offsets"))
        assert ln.tolist() == lengths, case["cite"]
        assert off.tolist() == offsets, case["cite"]


# ---------------------------------------------------------------- brute force

def _random_case(rng, kind, feat):
    s = int(rng.integers(0, 9))
    lengths = rng.integers(0, 7, size=s)
    lengths[rng.random(s) < 0.25] = 0
    base = int(rng.integers(0, 4))  # offsets[0] may be above zero
    offsets = np.concatenate([[base], base + np.cumsum(lengths)]).astype(np.int64)
    rows = int(offsets[-1]) + int(rng.integers(0, 3))  # rows past the last offset are never read
    if kind == "f32":
        # finite, no zeros (so Python's order equals the key order), many ties
        pool = np.array([-2.5, -1.0, -0.375, 0.125, 0.5, 1.0, 3.0, 1e-3, -7e-4, 6.5e3], dtype=np.float32)
        vals = pool[rng.integers(0, len(pool), size=(rows, feat))]
        vals = np.where(rng.random((rows, feat)) < 0.5, vals, rng.uniform(-4, 4, (rows, feat)).astype(np.float32))
        vals[vals == 0] = 0.25
    elif kind == "i32":
        vals = rng.integers(-(2 ** 31), 2 ** 31, size=(rows, feat), dtype=np.int64)
        vals[rng.random((rows, feat)) < 0.4] = rng.integers(-3, 3)
        vals = vals.astype(np.int32)
    else:
        vals = rng.integers(0, 2 ** 32, size=(rows, feat), dtype=np.uint64)
        vals[rng.random((rows, feat)) < 0.4] = rng.integers(0, 3)
        vals = vals.astype(np.uint32)
    return vals, offsets


def pin_brute_random(lib, cases=300, seed=1234):
    """Oracle == pure-Python brute force on tiny random inputs (F in 1,2,3,5)."""
    rng = np.random.default_rng(seed)
    for i in range(cases):
        kind = ("u32", "i32", "f32")[i % 3]
        feat = (1, 2, 3, 5)[(i // 3) % 4]
        vals, off = _random_case(rng, kind, feat)
        rows = vals.tolist()
        ops = ("sum", "min", "max") + (("mean",) if kind == "f32" else ())
        for op in ops:
            r = oracle.reduce(vals if feat > 1 else vals[:, 0], off, op, lib=lib)
            b_out, b_arg, b_exact = brute_ref.reduce(rows, off.tolist(), op, kind, feat)
            s = len(off) - 1
            if op in ("min", "max"):
                assert r.out.tolist() == b_out, (i, kind, op)
                assert r.arg.tolist() == b_arg, (i, kind, op)
            elif kind == "f32":
                for si in range(s):
                    for f in range(feat):
                        lo, hi = off[si], off[si + 1]
                        n = int(hi - lo)
                        ex = b_exact[si][f]
                        a = math.fsum(abs(float(vals[r, f])) for r in range(lo, hi))
                        scale = a / n if (op == "mean" and n) else a
                        assert abs(r.ref[si, f] - ex) <= 1e-13 * scale + 1e-300, (i, op, si, f)
                        assert abs(r.mag[si, f] - a) <= 1e-13 * a + 1e-300, (i, op, si, f)
                        # the float32 output is the double result rounded once
                        assert abs(float(r.out[si, f]) - ex) <= 2.0 ** -23 * abs(ex) + 1e-13 * scale + 1e-300, (i, op, si, f)
            else:
                assert r.out.tolist() == b_out, (i, kind, op)


# ---------------------------------------------------------------- library special cases

def pin_library_special_cases(lib, seed=7):
    """S = 1 is a global reduction; nonempty segments match numpy reduceat;
    F features are F independent columns; float sums match torch.segment_reduce."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(-1, 1, 5000).astype(np.float32)
    xi = rng.integers(-1000, 1001, 5000, dtype=np.int32)
    off1 = np.array([17, 4321], dtype=np.int64)
    seg = x[17:4321]
    r = oracle.reduce(x, off1, "sum", lib=lib)
    assert abs(r.ref[0, 0] - np.sum(seg, dtype=np.float64)) <= 1e-12 * np.abs(seg).sum()
    assert abs(r.mag[0, 0] - np.abs(seg).sum(dtype=np.float64)) <= 1e-12 * np.abs(seg).sum()
    for op, fn, afn in (("min", np.min, np.argmin), ("max", np.max, np.argmax)):
        for arr in (x, xi):
            r = oracle.reduce(arr, off1, op, lib=lib)
            assert r.out[0, 0] == fn(arr[17:4321]) and r.arg[0, 0] == 17 + afn(arr[17:4321]), op

    # many segments, some empty: reduceat on the nonempty ones
    lengths = rng.integers(0, 40, 300)
    lengths[rng.random(300) < 0.2] = 0
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    n = int(off[-1])
    vals = rng.integers(-50, 50, n, dtype=np.int32)
    ne = lengths > 0
    starts = off[:-1][ne]
    for op, ufunc in (("sum", np.add), ("min", np.minimum), ("max", np.maximum)):
        r = oracle.reduce(vals, off, op, lib=lib)
        want = ufunc.reduceat(vals.astype(np.int64) if op == "sum" else vals, starts)
        assert np.array_equal(r.out[ne, 0].astype(np.int64), want.astype(np.int64)), op
        assert (r.out[~ne, 0] == 0).all(), op

    # F columns are independent 1-D problems
    feat = 6
    v2 = rng.standard_normal((n, feat)).astype(np.float32)
    for op in ("sum", "min", "max", "mean"):
        r2 = oracle.reduce(v2, off, op, lib=lib)
        for f in range(feat):
            r1 = oracle.reduce(np.ascontiguousarray(v2[:, f]), off, op, lib=lib)
            assert np.array_equal(r2.out[:, f], r1.out[:, 0]), (op, f)
            if r1.arg is not None:
                assert np.array_equal(r2.arg[:, f], r1.arg[:, 0]), (op, f)

    # torch.segment_reduce (CPU), the library the graph-reduce README compares against
    import torch
    tv = torch.from_numpy(v2.astype(np.float64))
    tl = torch.from_numpy(lengths.astype(np.int64))
    r = oracle.reduce(v2, off, "sum", lib=lib)
    ts = torch.segment_reduce(tv, "sum", lengths=tl, axis=0, unsafe=True).numpy()
    assert np.allclose(r.ref, ts, rtol=0, atol=1e-12 * max(1.0, np.abs(v2).sum()))
    tm = torch.segment_reduce(tv, "mean", lengths=tl, axis=0, unsafe=True).numpy()
    rm = oracle.reduce(v2, off, "mean", lib=lib)
    tm = np.where(ne[:, None], tm, 0.0)
    assert np.allclose(rm.ref, tm, rtol=1e-12, atol=1e-12)
    for op in ("min", "max"):
        tmx = torch.segment_reduce(torch.from_numpy(v2), op, lengths=tl, axis=0, unsafe=True).numpy()
        rr = oracle.reduce(v2, off, op, lib=lib)
        assert np.array_equal(rr.out[ne], tmx[ne]), op


def pin_integer_valued_floats(lib, seed=11):
    """Integer-valued floats with small partial sums add exactly in any order,
    so the float32 result must equal a float64 numpy sum bit for bit."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, 300, 200)
    off = np.concatenate([[3], 3 + np.cumsum(lengths)]).astype(np.int64)
    vals = rng.integers(-3, 4, (int(off[-1]) + 5, 3)).astype(np.float32)
    r = oracle.reduce(vals, off, "sum", lib=lib)
    for s in range(200):
        want = vals[off[s]:off[s + 1]].astype(np.float64).sum(axis=0)
        assert np.array_equal(r.out[s], want.astype(np.float32)), s


def pin_wraparound(lib):
    """Integer sums are taken modulo 2^32 (closed form)."""
    off = np.array([0, 2, 4, 7], dtype=np.int64)
    u = np.array([0xFFFFFFFF, 2, 0x80000000, 0x80000000, 1, 2, 3], dtype=np.uint32)
    assert _col(oracle.reduce(u, off, "sum", lib=lib).out) == [1, 0, 6]
    i = np.array([2 ** 31 - 1, 1, -(2 ** 31), -1, -5, 2, 3], dtype=np.int32)
    assert _col(oracle.reduce(i, off, "sum", lib=lib).out) == [-(2 ** 31), 2 ** 31 - 1, 0]
    # u32 min/max compare unsigned, i32 signed
    assert _col(oracle.reduce(u, off, "max", lib=lib).out) == [0xFFFFFFFF, 0x80000000, 3]
    assert _col(oracle.reduce(i, off, "min", lib=lib).out) == [1, -(2 ** 31), -5]


def pin_mean(lib, seed=5):
    """mean = sum / length, empty -> 0 (graph-reduce README, 'API')."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, 30, 100)
    lengths[::7] = 0
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    v = rng.standard_normal((int(off[-1]), 2)).astype(np.float32)
    r = oracle.reduce(v, off, "mean", lib=lib)
    for s in range(100):
        if lengths[s] == 0:
            assert (r.out[s] == 0).all() and (r.ref[s] == 0).all()
        else:
            want = v[off[s]:off[s + 1]].astype(np.float64).mean(axis=0)
            assert np.allclose(r.ref[s], want, rtol=1e-13, atol=1e-15), s


# ---------------------------------------------------------------- order key and invariants

def _fbits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def pin_order_key(lib, seed=3):
    """The monotone key orders floats as numpy does (finite, distinct, nonzero),
    int32 as signed integers and uint32 as unsigned; -0.0 sorts just below +0.0
    and NaNs sit outside +-inf (the reading of the graph-reduce 'Method')."""
    rng = np.random.default_rng(seed)
    xs = np.unique(np.concatenate([rng.standard_normal(2000), rng.uniform(-1e30, 1e30, 500),
                                   [np.inf, -np.inf, 1e-40, -1e-40]]).astype(np.float32))
    xs = xs[xs != 0]
    keys = [oracle.order_key(_fbits(float(v)), "f32", lib=lib) for v in xs]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)
    kneg0 = oracle.order_key(0x80000000, "f32", lib=lib)
    kpos0 = oracle.order_key(0x00000000, "f32", lib=lib)
    kmin = oracle.order_key(_fbits(-1e-40), "f32", lib=lib)
    kmax = oracle.order_key(_fbits(1e-40), "f32", lib=lib)
    assert kmin < kneg0 < kpos0 < kmax
    assert oracle.order_key(0x7FC00000, "f32", lib=lib) > oracle.order_key(_fbits(np.inf), "f32", lib=lib)
    assert oracle.order_key(0xFFC00000, "f32", lib=lib) < oracle.order_key(_fbits(-np.inf), "f32", lib=lib)
    ints = np.unique(rng.integers(-(2 ** 31), 2 ** 31, 3000))
    ik = [oracle.order_key(int(v) & 0xFFFFFFFF, "i32", lib=lib) for v in ints]
    assert ik == sorted(ik)
    us = np.unique(rng.integers(0, 2 ** 32, 3000))
    assert [oracle.order_key(int(v), "u32", lib=lib) for v in us] == [int(v) for v in us]


def pin_minmax_invariants(lib, seed=9):
    """On tie-heavy data, every arg is gathered back, lies in its segment, has no
    better row in the segment and no earlier row with an equal value
    (graph-reduce README, 'Correctness')."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, 50, 400)
    off = np.concatenate([[5], 5 + np.cumsum(lengths)]).astype(np.int64)
    n = int(off[-1]) + 5
    for kind, vals in (("i32", rng.integers(-3, 3, (n, 2)).astype(np.int32)),
                       ("u32", rng.integers(0, 4, (n, 2)).astype(np.uint32)),
                       ("f32", rng.integers(-2, 3, (n, 2)).astype(np.float32) * np.float32(0.5) + np.float32(0.25))):
        for op in ("min", "max"):
            r = oracle.reduce(vals, off, op, lib=lib)
            for s in range(400):
                lo, hi = int(off[s]), int(off[s + 1])
                for f in range(2):
                    a = int(r.arg[s, f])
                    if lo == hi:
                        assert a == -1 and r.out[s, f] == 0
                        continue
                    assert lo <= a < hi, (kind, op, s)
                    col = vals[lo:hi, f]
                    assert r.out[s, f] == vals[a, f]
                    best = col.min() if op == "min" else col.max()
                    assert vals[a, f] == best, (kind, op, s)
                    assert not (col[: a - lo] == best).any(), (kind, op, s)


def pin_rle_groupby(lib, seed=13):
    """RLE equals itertools.groupby (adjacent runs) on random keys, and the
    offsets are the running sum of the lengths."""
    rng = np.random.default_rng(seed)
    for trial in range(40):
        n = int(rng.integers(0, 400))
        keys = np.repeat(rng.integers(0, 5, n), rng.integers(1, 6, n))[:n].astype(np.uint32)
        if trial % 4 == 0:
            keys = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
        v, ln, off, c = oracle.rle(keys, lib=lib)
        groups = [(k, len(list(g))) for k, g in itertools.groupby(keys.tolist())]
        assert v.tolist() == [k for k, _ in groups]
        assert ln.tolist() == [m for _, m in groups]
        assert off.tolist() == list(itertools.accumulate([0] + [m for _, m in groups]))
        bv, bl, bo = brute_ref.rle(keys.tolist())
        assert (v.tolist(), ln.tolist(), off.tolist()) == (bv, bl, bo)


# ---------------------------------------------------------------- scatter path

def _index_of_offsets(off):
    """The index vector of a CSR offsets array: row r -> the segment holding it
    (rows before offsets[0] or past offsets[-1] get -1, i.e. no output)."""
    n = int(off[-1])
    idx = np.full(n, -1, dtype=np.int64)
    for s in range(len(off) - 1):
        idx[int(off[s]):int(off[s + 1])] = s
    return idx


def pin_scatter_worked_example(lib):
    """The luma.gl worked example written as a destination index (graph-reduce
    README, 'Usage': the sorted edge list and its CSR pointer describe the same
    grouping), then with its rows shuffled: the values may not change."""
    g = _golden("segmented_reduction_worked_example.json")
    off = np.array(g["offsets"], dtype=np.int64)
    idx = _index_of_offsets(off)
    s = len(off) - 1
    assert oracle.offsets_from_index(idx, s, lib=lib).tolist() == off.tolist()
    perm = np.random.default_rng(0).permutation(len(idx))
    for kind in ("u32", "i32", "f32"):
        vals = np.array(g["values"], dtype=NP_T[kind])[: len(idx)]
        for op in ("sum", "min", "max"):
            r = oracle.scatter(vals, idx, s, op, lib=lib)
            assert _col(r.out) == g[op], (kind, op)
            if op != "sum":
                assert _col(r.arg) == g["derived"]["arg" + op], (kind, op)
            rp = oracle.scatter(vals[perm], idx[perm], s, op, lib=lib)
            assert _col(rp.out) == g[op], (kind, op, "shuffled")


def _random_scatter_case(rng, kind, feat):
    rows = int(rng.integers(0, 40))
    dim = int(rng.integers(0, 9))
    index = rng.integers(-2, dim + 3, rows).astype(np.int64)  # some rows fall outside
    pool = {"f32": lambda n: rng.choice(np.array([-2.5, -1.0, 0.5, 0.125, 3.0, 7e-4], np.float32), n),
            "i32": lambda n: rng.integers(-3, 3, n).astype(np.int32),
            "u32": lambda n: rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)}[kind]
    vals = pool(rows * feat).reshape(rows, feat)
    if kind == "u32":
        vals[rng.random((rows, feat)) < 0.5] = 7  # ties
    return vals, index, dim


def pin_scatter_brute(lib, cases=300, seed=4321):
    """Scatter oracle == pure-Python brute force on tiny random inputs with
    unsorted, repeated and out-of-range indices (F in 1, 2, 3)."""
    rng = np.random.default_rng(seed)
    for i in range(cases):
        kind = ("u32", "i32", "f32")[i % 3]
        feat = (1, 2, 3)[(i // 3) % 3]
        vals, index, dim = _random_scatter_case(rng, kind, feat)
        ops = ("sum", "min", "max") + (("mean",) if kind == "f32" else ())
        for op in ops:
            r = oracle.scatter(vals if feat > 1 else vals[:, 0], index, dim, op, lib=lib)
            b_out, b_arg, b_exact = brute_ref.scatter(vals.tolist(), index.tolist(), dim, op, kind, feat)
            if op in ("min", "max"):
                assert r.out.tolist() == b_out and r.arg.tolist() == b_arg, (i, kind, op)
            elif kind == "f32":
                for s in range(dim):
                    for f in range(feat):
                        ex = b_exact[s][f]
                        a = math.fsum(abs(float(vals[k, f])) for k in range(len(index)) if index[k] == s)
                        assert abs(r.ref[s, f] - ex) <= 1e-13 * a + 1e-300, (i, op, s, f)
                        assert abs(r.mag[s, f] - a) <= 1e-13 * a + 1e-300, (i, op, s, f)
                        assert abs(float(r.out[s, f]) - ex) <= 2.0 ** -23 * abs(ex) + 1e-13 * a + 1e-300, (i, op, s, f)
            else:
                assert r.out.tolist() == b_out, (i, kind, op)
        assert oracle.offsets_from_index(index, dim, lib=lib).tolist() == brute_ref.offsets_from_index(index.tolist(), dim)


def pin_scatter_library(lib, seed=17):
    """torch on the CPU, the baselines the graph-reduce README names: index_add_
    for sums, scatter_reduce(amax / amin, include_self=False) for values,
    torch.bincount + cumsum for the CSR pointer; and on a sorted index the
    scatter equals the segmented reduction over that pointer."""
    import torch
    rng = np.random.default_rng(seed)
    rows, dim, feat = 6000, 700, 3
    index = rng.integers(0, dim, rows).astype(np.int64)
    index[rng.random(rows) < 0.05] = dim + 5  # out of range: dropped before torch sees it
    keep = index < dim
    v = rng.standard_normal((rows, feat)).astype(np.float32)
    ti = torch.from_numpy(index[keep])
    tv = torch.from_numpy(v[keep].astype(np.float64))
    want = torch.zeros(dim, feat, dtype=torch.float64).index_add_(0, ti, tv).numpy()
    r = oracle.scatter(v, index, dim, "sum", lib=lib)
    assert np.allclose(r.ref, want, rtol=0, atol=1e-12 * max(1.0, np.abs(v).sum()))
    counts = torch.bincount(ti, minlength=dim).numpy()
    rm = oracle.scatter(v, index, dim, "mean", lib=lib)
    assert np.allclose(rm.ref, np.where(counts[:, None] > 0, want / np.maximum(counts, 1)[:, None], 0.0),
                       rtol=1e-12, atol=1e-14)
    for op, red in (("min", "amin"), ("max", "amax")):
        for arr in (v, rng.integers(-50, 50, (rows, feat)).astype(np.int32)):
            tgt = torch.zeros(dim, feat, dtype=torch.from_numpy(arr).dtype)
            t = tgt.scatter_reduce(0, ti[:, None].expand(-1, feat), torch.from_numpy(arr[keep]), red,
                                   include_self=False).numpy()
            rr = oracle.scatter(arr, index, dim, op, lib=lib)
            assert np.array_equal(rr.out, t), (op, arr.dtype)
            # the arg is gathered back and is the lowest row among equals
            for s in range(0, dim, 7):
                for f in range(feat):
                    members = np.nonzero(index == s)[0]
                    a = int(rr.arg[s, f])
                    if members.size == 0:
                        assert a == -1
                        continue
                    col = arr[members, f]
                    best = col.min() if op == "min" else col.max()
                    assert index[a] == s and arr[a, f] == best and a == members[col == best][0]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    assert np.array_equal(oracle.offsets_from_index(index, dim, lib=lib), off)
    # sorted index: scatter == segmented reduction over the counted pointer
    order = np.argsort(index, kind="stable")
    si, sv = index[order], v[order]
    soff = oracle.offsets_from_index(si, dim, lib=lib)
    for op in ("sum", "min", "max", "mean"):
        a = oracle.scatter(sv, si, dim, op, lib=lib)
        b = oracle.reduce(sv[: int(soff[-1])], soff, op, lib=lib)
        assert np.array_equal(a.out, b.out), op
        if a.arg is not None:
            assert np.array_equal(a.arg, b.arg), op


# ---------------------------------------------------------------- unique and start flags

def pin_unique(lib, seed=19):
    """GPUUnique (luma.gl RLE page, 'GPUUnique'): the printed RLE examples'
    values, then itertools.groupby, numpy's adjacent-difference mask and the
    brute-force definition on random keys (long runs and all-distinct)."""
    g = _golden("run_length_encode_examples.json")
    for case in g["cases"]:
        v, c = oracle.unique(np.array(case["input"], dtype=np.uint32), lib=lib)
        assert v.tolist() == case["values"] and c == len(case["values"]), case["cite"]
    rng = np.random.default_rng(seed)
    for trial in range(40):
        n = int(rng.integers(0, 500))
        keys = np.repeat(rng.integers(0, 4, n), rng.integers(1, 7, n))[:n].astype(np.uint32)
        if trial % 3 == 0:
            keys = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
        v, c = oracle.unique(keys, lib=lib)
        assert v.tolist() == [k for k, _ in itertools.groupby(keys.tolist())]
        if n:
            assert np.array_equal(v, keys[np.concatenate([[True], keys[1:] != keys[:-1]])])
        assert v.tolist() == brute_ref.unique(keys.tolist()) and c == v.size


def pin_offsets_from_flags(lib, seed=23):
    """Offsets from segment-start flags: the printed layouts (tests/golden),
    numpy flatnonzero, brute force, and the RLE identity: the run-start flags
    of any key vector give the RLE offsets."""
    g = _golden("segment_start_flags.json")
    for case in g["cases"]:
        off, c = oracle.offsets_from_flags(np.array(case["flags"], dtype=np.uint32), lib=lib)
        assert off.tolist() == case["offsets"] and c == case["count"], case["cite"]
    rng = np.random.default_rng(seed)
    for trial in range(40):
        n = int(rng.integers(0, 600))
        flags = (rng.random(n) < rng.choice([0.0, 0.02, 0.3, 1.0])).astype(np.uint32)
        flags *= rng.integers(1, 2 ** 32, n, dtype=np.uint64).astype(np.uint32) | np.uint32(2)  # any nonzero word
        off, c = oracle.offsets_from_flags(flags, lib=lib)
        assert off.tolist() == np.flatnonzero(flags).tolist() + [n]
        assert off.tolist() == brute_ref.offsets_from_flags(flags.tolist()) and c == off.size - 1
        keys = np.repeat(rng.integers(0, 3, n), rng.integers(1, 5, n))[:n].astype(np.uint32)
        heads = np.ones(n, dtype=np.uint32)
        if n:
            heads[1:] = keys[1:] != keys[:-1]
        _, _, roff, rc = oracle.rle(keys, lib=lib)
        off2, c2 = oracle.offsets_from_flags(heads, lib=lib)
        assert off2.tolist() == roff.tolist() and c2 == rc


# ---------------------------------------------------------------- segmented scan

def pin_scan_against_printed_reduction(lib):
    """The inclusive scan ends every segment on the printed segmented sum /
    min / max (luma.gl GPUSegmentedReduction, 'What is segmented reduction?');
    the exclusive scan starts every segment at 0 and lags the inclusive one by
    a row."""
    g = _golden("segmented_reduction_worked_example.json")
    off = np.array(g["offsets"], dtype=np.int64)
    for kind in ("u32", "i32", "f32"):
        vals = np.array(g["values"], dtype=NP_T[kind])
        for op in ("sum", "min", "max"):
            inc = oracle.scan(vals, off, op, exclusive=False, lib=lib).out[:, 0]
            exc = oracle.scan(vals, off, op, exclusive=True, lib=lib).out[:, 0]
            assert [inc[int(off[s + 1]) - 1] for s in range(3)] == g[op], (kind, op)
            for s in range(3):
                lo, hi = int(off[s]), int(off[s + 1])
                assert exc[lo] == 0 and np.array_equal(exc[lo + 1:hi], inc[lo:hi - 1]), (kind, op, s)


def pin_scan_brute(lib, cases=200, seed=29):
    """Scan oracle == brute force (each prefix recomputed from scratch) on tiny
    random inputs with empty segments, offsets[0] > 0 and unread rows."""
    rng = np.random.default_rng(seed)
    for i in range(cases):
        kind = ("u32", "i32", "f32")[i % 3]
        feat = (1, 2, 3)[(i // 3) % 3]
        vals, off = _random_case(rng, kind, feat)
        rows = vals.tolist()
        for op in ("sum", "min", "max"):
            for exclusive in (False, True):
                r = oracle.scan(vals if feat > 1 else vals[:, 0], off, op, exclusive, fill=7, lib=lib)
                b = brute_ref.scan(rows, off.tolist(), op, kind, feat, exclusive)
                for q in range(vals.shape[0]):
                    if q not in b:
                        assert (r.out[q] == 7).all(), (i, q)  # rows outside the segments are not written
                        continue
                    outs, exact = b[q]
                    if exact is None:
                        assert r.out[q].tolist() == outs, (i, kind, op, exclusive, q)
                    else:
                        for f in range(feat):
                            assert abs(r.ref[q, f] - exact[f]) <= 1e-13 * r.mag[q, f] + 1e-300, (i, q, f)
                            assert float(r.out[q, f]) == outs[f] or \
                                abs(float(r.out[q, f]) - exact[f]) <= 2.0 ** -24 * abs(exact[f]) + 1e-13 * r.mag[q, f]


def pin_scan_library(lib, seed=31):
    """numpy per segment: cumsum (int64 mod 2^32, float64), minimum /
    maximum.accumulate; the last inclusive row of each segment equals the
    segmented reduction."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, 60, 300)
    lengths[rng.random(300) < 0.2] = 0
    off = np.concatenate([[4], 4 + np.cumsum(lengths)]).astype(np.int64)
    n = int(off[-1]) + 3
    cases = (("i32", rng.integers(-(2 ** 31), 2 ** 31, (n, 2)).astype(np.int32)),
             ("u32", rng.integers(0, 2 ** 32, (n, 2), dtype=np.uint64).astype(np.uint32)),
             ("f32", rng.standard_normal((n, 2)).astype(np.float32)))
    for kind, vals in cases:
        for op in ("sum", "min", "max"):
            inc = oracle.scan(vals, off, op, False, lib=lib)
            red = oracle.reduce(vals, off, op, lib=lib)
            for s in range(300):
                lo, hi = int(off[s]), int(off[s + 1])
                if lo == hi:
                    continue
                seg = vals[lo:hi]
                if op == "sum" and kind == "f32":
                    want = np.cumsum(seg.astype(np.float64), axis=0)
                    assert np.allclose(inc.ref[lo:hi], want, rtol=1e-12, atol=1e-12), (kind, s)
                    assert abs(inc.ref[hi - 1, 0] - red.ref[s, 0]) <= 1e-12 * red.mag[s, 0] + 1e-300
                    continue
                if op == "sum":
                    want = (np.cumsum(seg.astype(np.int64), axis=0) % (1 << 32)).astype(np.uint64)
                    got = inc.out[lo:hi].view(np.uint32).astype(np.uint64)
                else:
                    acc = np.minimum.accumulate if op == "min" else np.maximum.accumulate
                    want, got = acc(seg, axis=0), inc.out[lo:hi]
                assert np.array_equal(got, want), (kind, op, s)
                assert np.array_equal(inc.out[hi - 1].view(np.uint32), red.out[s].view(np.uint32)), (kind, op, s)


# ---------------------------------------------------------------- lower-bound search

def _lb_case(rng, kind, segs, vmax, qmax, order=False, stride=1):
    """Sorted value segments (optionally reached through a permutation order
    vector and a stride) and sorted queries per segment."""
    vcs = rng.integers(0, vmax + 1, segs)
    qcs = rng.integers(0, qmax + 1, segs)
    vo = (np.cumsum(vcs) - vcs).astype(np.int64)
    qo = (np.cumsum(qcs) - qcs).astype(np.int64)
    nv, nq = int(vcs.sum()), int(qcs.sum())
    if kind == "f32":
        pool = rng.standard_normal(nv).astype(np.float32)
        pool[rng.random(nv) < 0.3] = np.float32(0.5)  # duplicates
        qs = rng.standard_normal(nq).astype(np.float32) * np.float32(1.3)
        qs[rng.random(nq) < 0.2] = np.float32(0.5)
    else:
        pool = rng.integers(0, 50, nv).astype(np.uint32)
        pool[rng.random(nv) < 0.1] = np.uint32(0xFFFFFFF0)
        qs = rng.integers(0, 52, nq).astype(np.uint32)
        qs[rng.random(nq) < 0.05] = np.uint32(0xFFFFFFFF)
    for s in range(segs):
        pool[vo[s]:vo[s] + vcs[s]].sort()
        qs[qo[s]:qo[s] + qcs[s]].sort()
    seg = np.stack([vo, vcs, qo, qcs], axis=1).astype(np.int64)
    ordv = None
    stored = pool
    if order:
        perm = rng.permutation(nv).astype(np.uint32)  # stored row of search position p
        stored = np.empty_like(pool)
        stored[perm] = pool
        ordv = perm
    if stride > 1:
        wide = np.zeros(nv * stride, dtype=pool.dtype)
        wide[::stride] = stored
        stored = wide
    return stored, qs, seg, ordv, pool


def pin_lower_bounds_library(lib, seed=37):
    """Every answer equals numpy.searchsorted(side='left') on its segment and
    bisect.bisect_left, directly, through an order vector, and strided."""
    import bisect
    rng = np.random.default_rng(seed)
    for trial in range(60):
        kind = ("u32", "f32")[trial % 2]
        order, stride = bool(trial % 3 == 1), (1, 1, 3)[trial % 3]
        stored, qs, seg, ordv, pool = _lb_case(rng, kind, int(rng.integers(1, 12)), 60, 70, order, stride)
        out, word = oracle.lower_bounds(stored, qs, seg, stride=stride, order=ordv,
                                        value_count=pool.shape[0] if stride > 1 else None, lib=lib)
        assert word == 0, trial
        for vo, vc, qo, qc in seg.tolist():
            v = pool[vo:vo + vc]
            want = vo + np.searchsorted(v, qs[qo:qo + qc], side="left")
            assert np.array_equal(out[qo:qo + qc], want), (trial, kind, order, stride)
            vl = v.tolist()
            for k in range(qc):
                assert out[qo + k] == vo + bisect.bisect_left(vl, qs[qo + k].item())


def pin_lower_bounds_brute(lib, seed=41):
    """Tiny cases against the scan-from-the-left definition (brute_ref)."""
    rng = np.random.default_rng(seed)
    for trial in range(150):
        kind = ("u32", "f32")[trial % 2]
        stored, qs, seg, _, pool = _lb_case(rng, kind, int(rng.integers(0, 5)), 9, 9)
        out, word = oracle.lower_bounds(stored, qs, seg, tile=int(rng.integers(1, 5)), lib=lib)
        for vo, vc, qo, qc in seg.tolist():
            for k in range(qc):
                assert out[qo + k] == vo + brute_ref.lower_bound(pool[vo:vo + vc].tolist(), qs[qo + k].item())


def pin_lower_bounds_validation(lib):
    """The validation word of the galloping-search page ('Validation'), bit by
    bit, on constructed inputs."""
    v = np.arange(10, dtype=np.float32)
    q = np.array([2.5, 1.0, 7.0, 3.0, np.nan, 4.0, 5.0, 8.0, 9.5, np.inf], dtype=np.float32)
    # bit 4: a query below its predecessor inside a tile; the answer stays exact
    out, w = oracle.lower_bounds(v, q[:4], np.array([[0, 10, 0, 4]]), tile=4, lib=lib)
    assert w == 4 and out.tolist() == [3, 1, 7, 3]
    # ... but not across a tile boundary (tiles of 1 and of 2 here)
    out, w = oracle.lower_bounds(v, q[:2], np.array([[0, 10, 0, 2]]), tile=1, lib=lib)
    assert w == 0 and out.tolist() == [3, 1]
    out, w = oracle.lower_bounds(v, q[1:3], np.array([[0, 10, 0, 2]]), tile=1, lib=lib)
    assert w == 0
    # bit 8: a non-finite query stops the rest of its tile; the next tile runs
    out, w = oracle.lower_bounds(v, q[3:10], np.array([[0, 10, 0, 7]]), tile=3, lib=lib)
    assert w == 8 and out.tolist() == [3, -7, -7, 5, 8, 10, -7]
    # bit 1: value range outside the view; bit 2: query range outside, or above capacity
    out, w = oracle.lower_bounds(v, q[:3], np.array([[5, 6, 0, 3]]), lib=lib)
    assert w == 1 and (out == -7).all()
    out, w = oracle.lower_bounds(v, q[:3], np.array([[0, 10, 1, 3]]), lib=lib)
    assert w == 2 and (out == -7).all()
    out, w = oracle.lower_bounds(v, q[:3], np.array([[0, 10, 0, 3]]), max_qc=2, lib=lib)
    assert w == 2 and (out == -7).all()
    out, w = oracle.lower_bounds(v, q[:3], np.array([[-1, 2, 0, 3], [0, 10, 0, 1]]), lib=lib)
    assert w == 1 and out.tolist() == [3, -7, -7]
    # empty segments are valid; preserve ORs into the old word
    out, w = oracle.lower_bounds(v, q[:1], np.array([[4, 0, 0, 1], [0, 0, 1, 0]]), validation=16, lib=lib)
    assert w == 0 and out.tolist() == [4]
    out, w = oracle.lower_bounds(v, q[:2], np.array([[0, 10, 0, 2]]), tile=2, validation=16, preserve=True, lib=lib)
    assert w == 20
    # uint32 compares unsigned
    vu = np.array([1, 5, 0x80000000, 0xFFFFFFFF], dtype=np.uint32)
    out, w = oracle.lower_bounds(vu, np.array([0x7FFFFFFF, 0xFFFFFFFF], np.uint32), np.array([[0, 4, 0, 2]]), lib=lib)
    assert w == 0 and out.tolist() == [2, 3]


ALL_PINS = [
    pin_lower_bounds_library,
    pin_lower_bounds_brute,
    pin_lower_bounds_validation,
    pin_scan_against_printed_reduction,
    pin_scan_brute,
    pin_scan_library,
    pin_unique,
    pin_offsets_from_flags,
    pin_scatter_worked_example,
    pin_scatter_brute,
    pin_scatter_library,
    pin_worked_example,
    pin_empty_segments,
    pin_rle_examples,
    pin_brute_random,
    pin_library_special_cases,
    pin_integer_valued_floats,
    pin_wraparound,
    pin_mean,
    pin_order_key,
    pin_minmax_invariants,
    pin_rle_groupby,
]
