"""Seeded synthetic inputs shaped like the workloads the pages describe.

This module only draws inputs; it holds none of the method's arithmetic and
is the one piece shared by the oracle side and the HIP side.  Every draw uses
``numpy.random.default_rng(seed)`` with a fixed draw order, so a seed fixes
the data bit for bit on any machine.  Offsets are built from the drawn
lengths with ``numpy.cumsum`` (the same construction the graph-reduce README
shows in its usage example with bincount + cumsum).

Configurations (sizes are decimal unless written as powers of two):

  small     1-D float32 / int32, 4,096 segments, lengths uniform in [0, 64]
            plus 1.5 % forced empty (about 3 % empty in all), values
            uniform[-1, 1] / integers in [-1000, 1000].
  message   graph message passing: 1,000,000 destination-sorted rows x 64
            float32 normal(0, 1) into 10,000 segments; lengths multinomial
            with mean 100 (the graph-reduce README's 1M x 64 -> 10,000 row).
  rle       16,000,000 uint32 keys drawn Zipf(s = 1.1) over 2^20 distinct
            values (truncated pmf, inverse CDF), mapped through a seeded
            permutation, sorted; payloads uint32 uniform (sums wrap) and
            int32 over the full range.
  skew      50,000,000 float32 uniform[0, 1) over 1,000,000 segments: 10 %
            empty, one 5,000,000-row segment, the rest Pareto(1.5) lengths
            scaled to the remaining rows.
  powerlaw  2,000,000 nodes, 32,000,000 destination-sorted edges, in-degree
            Lomax/Pareto-II (alpha = 2) capped at 200,000 with one hub of
            exactly 200,000, F = 32 float32 normal(0, 1).
  search    lower-bound queries over segmented sorted values, shaped like the
            galloping-search page's uses (sampled time domains, repeated
            threshold lookup) with its Usage defaults (maximumQueryCount
            2049, 32 queries per tile): 8,192 segments, each a float32 time
            axis of uniform[0, 4096] stamps (cumulative exponential gaps),
            and uniform[0, 2049] sorted queries drawn over the segment's time
            span widened by 5 % on both sides.
  scatter   the message rows in edge order: 1,000,000 rows x F float32
            normal(0, 1) with an int64 destination index drawn uniformly over
            10,000 outputs, unsorted (the graph-reduce README's scatter_*
            usage; its measured table has this 1M -> 10,000 shape at F = 16
            and F = 64).
"""
from __future__ import annotations

import numpy as np


def _offsets(lengths, base=0):
    return np.concatenate([[base], base + np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int64)


def small(seed=0):
    rng = np.random.default_rng(seed)
    s = 4096
    lengths = rng.integers(0, 65, s)
    lengths[rng.random(s) < 0.015] = 0
    off = _offsets(lengths)
    n = int(off[-1])
    return {
        "name": "small-1d-4096seg",
        "offsets": off,
        "f32": rng.uniform(-1, 1, n).astype(np.float32),
        "i32": rng.integers(-1000, 1001, n, dtype=np.int32),
    }


def message(seed=0, feat=64):
    rng = np.random.default_rng(seed)
    s, n = 10_000, 1_000_000
    lengths = rng.multinomial(n, np.full(s, 1.0 / s))
    off = _offsets(lengths)
    values = rng.standard_normal((n, feat), dtype=np.float32)
    return {"name": f"message-1Mx{feat}-10Kseg", "offsets": off, "f32": values}


def rle_keys(seed=0, n=16_000_000, distinct=2 ** 20, s_exp=1.1):
    rng = np.random.default_rng(seed)
    ranks = np.arange(1, distinct + 1, dtype=np.float64)
    pmf = ranks ** (-s_exp)
    cdf = np.cumsum(pmf)
    cdf /= cdf[-1]
    u = rng.random(n)
    r = np.minimum(np.searchsorted(cdf, u, side="right"), distinct - 1)
    perm = rng.permutation(distinct).astype(np.uint32)
    keys = np.sort(perm[r])
    pay_u32 = rng.integers(0, 2 ** 32, n, dtype=np.uint32)
    pay_i32 = rng.integers(-(2 ** 31), 2 ** 31, n, dtype=np.int32)
    return {"name": f"rle-{n // 1_000_000}M-zipf1.1", "keys": keys, "u32": pay_u32, "i32": pay_i32}


def _largest_remainder(x, target):
    base = np.floor(x).astype(np.int64)
    rem = int(target - base.sum())
    if rem > 0:
        frac = x - base
        top = np.argsort(-frac, kind="stable")[:rem]
        base[top] += 1
    return base


def skew(seed=0, values=True):
    rng = np.random.default_rng(seed)
    s, n, hub_len, n_empty = 1_000_000, 50_000_000, 5_000_000, 100_000
    empty = rng.choice(s, n_empty, replace=False)
    mask = np.ones(s, dtype=bool)
    mask[empty] = False
    nonempty = np.flatnonzero(mask)
    hub = int(nonempty[rng.integers(0, nonempty.size)])
    others = nonempty[nonempty != hub]
    w = 1.0 + rng.pareto(1.5, others.size)
    lengths = np.zeros(s, dtype=np.int64)
    lengths[others] = _largest_remainder(w / w.sum() * (n - hub_len), n - hub_len)
    lengths[hub] = hub_len
    off = _offsets(lengths)
    out = {"name": "skew-50M-1Mseg", "offsets": off, "hub": hub}
    if values:
        out["f32"] = rng.random(n, dtype=np.float32)
    return out


def powerlaw(seed=0, values=True, feat=32):
    rng = np.random.default_rng(seed)
    s, n, cap = 2_000_000, 32_000_000, 200_000
    hub = int(rng.integers(0, s))
    x = rng.pareto(2.0, s - 1)
    target = n - cap

    def total(c):
        return int(np.minimum(np.floor(c * x), cap).sum())

    lo, hi = 0.0, 1.0
    while total(hi) < target:
        hi *= 2
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if total(mid) <= target:
            lo = mid
        else:
            hi = mid
    scaled = lo * x
    deg = np.minimum(np.floor(scaled), cap).astype(np.int64)
    rem = target - int(deg.sum())
    if rem > 0:
        frac = np.where(deg < cap, scaled - np.floor(scaled), -1.0)
        top = np.argsort(-frac, kind="stable")[:rem]
        deg[top] += 1
    lengths = np.insert(deg, hub, cap)
    off = _offsets(lengths)
    out = {"name": f"powerlaw-32Mx{feat}-2Mseg", "offsets": off, "hub": hub, "scale": lo}
    if values:
        out["f32"] = rng.standard_normal((n, feat), dtype=np.float32)
    return out


def scatter(seed=0, feat=64, rows=1_000_000, dim=10_000):
    rng = np.random.default_rng(seed)
    index = rng.integers(0, dim, rows, dtype=np.int64)
    values = rng.standard_normal((rows, feat), dtype=np.float32)
    tag = f"{dim // 1000}K" if dim >= 1000 else str(dim)
    return {"name": f"scatter-{rows // 1_000_000}Mx{feat}-{tag}dst", "index": index, "dim": dim,
            "f32": values}


def search(seed=0, segments=8_192, max_values=4_096, max_queries=2_049):
    rng = np.random.default_rng(seed)
    vcs = rng.integers(0, max_values + 1, segments)
    qcs = rng.integers(0, max_queries + 1, segments)
    nv, nq = int(vcs.sum()), int(qcs.sum())
    gaps = rng.exponential(1.0, nv).astype(np.float32)
    values = np.empty(nv, dtype=np.float32)
    queries = np.empty(nq, dtype=np.float32)
    vo = np.cumsum(vcs) - vcs
    qo = np.cumsum(qcs) - qcs
    u = rng.random(nq)
    for s in range(segments):
        v = np.cumsum(gaps[vo[s]:vo[s] + vcs[s]], dtype=np.float64)
        values[vo[s]:vo[s] + vcs[s]] = v.astype(np.float32)
        span = float(v[-1]) if vcs[s] else 1.0
        lo, hi = -0.05 * span, 1.05 * span
        queries[qo[s]:qo[s] + qcs[s]] = np.sort(lo + (hi - lo) * u[qo[s]:qo[s] + qcs[s]]).astype(np.float32)
    # (rounding a nondecreasing float64 sum to float32 keeps it nondecreasing)
    segs = np.stack([vo, vcs, qo, qcs], axis=1).astype(np.int64)
    return {"name": f"search-{segments // 1024}Kseg", "values": values, "queries": queries,
            "segments": segs, "max_query_count": max_queries, "queries_per_tile": 32}


CONFIGS = {"small": small, "message": message, "rle": rle_keys, "skew": skew, "powerlaw": powerlaw,
           "scatter": scatter, "search": search}


# ---------------------------------------------------------------- test-sized cases

def ragged(seed, segments, mean_len, feat=1, dtype="f32", empty_frac=0.1, base=0,
           long_segment=0, tail_rows=0, values="normal"):
    """A ragged case for parity tests: lengths uniform in [0, 2 * mean_len],
    a fraction forced empty, optionally one long segment, offsets starting at
    ``base`` and ``tail_rows`` unread rows after the last offset.

    ``values``: "normal" (float32 normal(0,1) / wide integers), "ties"
    (few distinct values, for tie-breaking) or "intfloat" (small integers as
    float32, whose sums are exact in any order)."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, 2 * mean_len + 1, segments) if segments else np.zeros(0, np.int64)
    if segments:
        lengths[rng.random(segments) < empty_frac] = 0
        if long_segment:
            lengths[int(rng.integers(0, segments))] = long_segment
    off = _offsets(lengths, base)
    rows = int(off[-1]) + tail_rows
    shape = (rows,) if feat == 1 else (rows, feat)
    if values == "ties":
        v = rng.integers(-2, 3, shape)
        arr = {"f32": (v * 0.5).astype(np.float32), "i32": v.astype(np.int32),
               "u32": (v + 2).astype(np.uint32)}[dtype]
    elif values == "intfloat":
        arr = rng.integers(-3, 4, shape).astype(np.float32)
    elif dtype == "f32":
        arr = rng.standard_normal(shape, dtype=np.float32)
    elif dtype == "i32":
        arr = rng.integers(-(2 ** 31), 2 ** 31, shape, dtype=np.int32)
    else:
        arr = rng.integers(0, 2 ** 32, shape, dtype=np.uint32)
    return off, arr


def scatter_case(seed, rows, dim, feat=1, dtype="f32", order="random", out_of_range=0.0, values="normal"):
    """An index-addressed case for the scatter tests.

    ``order``: "random" (uniform over [0, dim)), "sorted" (the same, sorted),
    "runs" (runs of 1..40 rows sharing a random destination) or "one" (every
    row to output 0).  A fraction ``out_of_range`` of the rows is then sent to
    -1, dim or 2^40 (rows that reach no output).  ``values`` as in ragged."""
    rng = np.random.default_rng(seed)
    hi = max(dim, 1)
    if order == "runs":
        lens = rng.integers(1, 41, rows + 1)
        dest = rng.integers(0, hi, lens.size)
        index = np.repeat(dest, lens)[:rows].astype(np.int64)
    elif order == "one":
        index = np.zeros(rows, dtype=np.int64)
    else:
        index = rng.integers(0, hi, rows, dtype=np.int64)
        if order == "sorted":
            index.sort()
    if out_of_range > 0 and rows:
        bad = rng.random(rows) < out_of_range
        index[bad] = rng.choice(np.array([-1, dim, 2 ** 40], dtype=np.int64), int(bad.sum()))
    shape = (rows,) if feat == 1 else (rows, feat)
    if values == "ties":
        v = rng.integers(-2, 3, shape)
        arr = {"f32": (v * 0.5).astype(np.float32), "i32": v.astype(np.int32),
               "u32": (v + 2).astype(np.uint32)}[dtype]
    elif dtype == "f32":
        arr = rng.standard_normal(shape, dtype=np.float32)
    elif dtype == "i32":
        arr = rng.integers(-(2 ** 31), 2 ** 31, shape, dtype=np.int32)
    else:
        arr = rng.integers(0, 2 ** 32, shape, dtype=np.uint32)
    return index, arr
