"""Brute-force reference in pure Python, used only to pin the oracle.

It is written independently of ``oracle/oracle.c``: Python integers and
``math.fsum`` (the correctly rounded sum) instead of fixed-width arithmetic,
Python's own float ordering instead of the monotone bit key, and
``min``/``max`` over (value, row) tuples for the tie rule.  It only accepts
inputs where Python's float order and the key order agree (finite floats, no
mix of -0.0 and +0.0), which the callers guarantee.

Semantics followed (luma.gl GPUSegmentedReduction page, "Contract";
graph-reduce README, "API" and "Correctness"): segment s covers rows
[offsets[s], offsets[s+1]); sum/min/max/mean per feature; empty segments give
0 (and arg -1); min/max ties go to the lower row.
"""
from __future__ import annotations

import math
import struct


def _f32(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]


def _round_f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def reduce(rows, offsets, op, kind, feat):
    """rows: list of lists (rows x feat) of Python ints (u32/i32) or floats (f32).

    Returns (out, arg, exact) as lists of lists [S][F]; ``exact`` holds the
    correctly rounded float sum (or mean) for float inputs, else None.
    """
    out, arg, exact = [], [], []
    for s in range(len(offsets) - 1):
        lo, hi = offsets[s], offsets[s + 1]
        o_row, a_row, e_row = [], [], []
        for f in range(feat):
            col = [(rows[r][f], r) for r in range(lo, hi)]
            if op in ("sum", "mean"):
                if kind == "f32":
                    total = math.fsum(v for v, _ in col)
                    val = total / (hi - lo) if (op == "mean" and hi > lo) else (total if op == "sum" else 0.0)
                    e_row.append(val)
                    o_row.append(_round_f32(val))
                else:
                    total = sum(v for v, _ in col) % (1 << 32)
                    if kind == "i32" and total >= (1 << 31):
                        total -= 1 << 32
                    o_row.append(total)
                a_row.append(None)
            else:
                if not col:
                    o_row.append(0)
                    a_row.append(-1)
                    continue
                # (value, row) tuples: the smallest/largest value, then the lowest row.
                if op == "min":
                    v, r = min(col)
                else:
                    v, r = max(col, key=lambda t: (t[0], -t[1]))
                o_row.append(v)
                a_row.append(r)
        out.append(o_row)
        arg.append(a_row)
        exact.append(e_row)
    return out, arg, (exact if kind == "f32" else None)


def rle(keys):
    """Adjacent runs by definition: a run continues while the next key equals it."""
    values, lengths = [], []
    for k in keys:
        if values and values[-1] == k and lengths:
            lengths[-1] += 1
        else:
            values.append(k)
            lengths.append(1)
    offsets = [0]
    for ln in lengths:
        offsets.append(offsets[-1] + ln)
    return values, lengths, offsets


def scatter(rows, index, dim_size, op, kind, feat):
    """Scatter by definition (graph-reduce README, "API"): output s gathers the
    rows r with index[r] == s, in row order; indices outside [0, dim_size)
    belong to no output.  Same result conventions as ``reduce``."""
    members = [[] for _ in range(dim_size)]
    for r, s in enumerate(index):
        if 0 <= s < dim_size:
            members[s].append(r)
    out, arg, exact = [], [], []
    for s in range(dim_size):
        o_row, a_row, e_row = [], [], []
        for f in range(feat):
            col = [(rows[r][f], r) for r in members[s]]
            n = len(col)
            if op in ("sum", "mean"):
                if kind == "f32":
                    total = math.fsum(v for v, _ in col)
                    val = total / n if (op == "mean" and n) else (total if op == "sum" else 0.0)
                    e_row.append(val)
                    o_row.append(_round_f32(val))
                else:
                    total = sum(v for v, _ in col) % (1 << 32)
                    if kind == "i32" and total >= (1 << 31):
                        total -= 1 << 32
                    o_row.append(total)
                a_row.append(None)
            elif not col:
                o_row.append(0)
                a_row.append(-1)
            else:
                # (value, row) tuples: the extreme value, then the lowest row
                best = min(col) if op == "min" else max(col, key=lambda t: (t[0], -t[1]))
                o_row.append(best[0])
                a_row.append(best[1])
        out.append(o_row)
        arg.append(a_row)
        exact.append(e_row)
    return out, arg, (exact if kind == "f32" else None)


def offsets_from_index(index, dim_size):
    """Counting by definition: offsets[s] = #{r : 0 <= index[r] < s}."""
    return [sum(1 for x in index if 0 <= x < s) for s in range(dim_size + 1)]


def unique(keys):
    """Adjacent distinct values by definition: keep a key when it differs from the last kept one."""
    out = []
    for k in keys:
        if not out or out[-1] != k:
            out.append(k)
    return out


def offsets_from_flags(flags):
    """Segment starts by definition: every position with a nonzero flag, then the length."""
    return [i for i, f in enumerate(flags) if f] + [len(flags)]


def scan(rows, offsets, op, kind, feat, exclusive):
    """Segmented prefix by definition: for every row, the op over the rows of
    its segment before it (exclusive; nothing -> 0) or up to it (inclusive),
    recomputed from scratch with math.fsum / Python ints / min / max.
    Returns {row: (list over features of outputs, list of exact float prefixes or None)}."""
    res = {}
    for s in range(len(offsets) - 1):
        lo, hi = offsets[s], offsets[s + 1]
        for r in range(lo, hi):
            upto = range(lo, r) if exclusive else range(lo, r + 1)
            outs, exact = [], []
            for f in range(feat):
                col = [rows[q][f] for q in upto]
                if op == "sum":
                    if kind == "f32":
                        t = math.fsum(col)
                        exact.append(t)
                        outs.append(_round_f32(t))
                    else:
                        t = sum(col) % (1 << 32)
                        if kind == "i32" and t >= (1 << 31):
                            t -= 1 << 32
                        outs.append(t)
                else:
                    outs.append((min(col) if op == "min" else max(col)) if col else 0)
            res[r] = (outs, exact if kind == "f32" and op == "sum" else None)
    return res


def lower_bound(seq, q):
    """First index whose element is not less than q (len(seq) if none), by scanning."""
    for i, v in enumerate(seq):
        if not v < q:
            return i
    return len(seq)
