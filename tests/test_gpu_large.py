"""Inputs past 2^31 rows and past 4 GiB (GPU only).

Values follow a closed form, generated on the device: element (r, f) is
((m r + f) mod 7) - 3 (m = F mod 7 is the step of the flattened index r F + f
modulo 7, invertible for the widths used), so every full period of 7 rows
sums to zero and each segment's sum, extrema and their first rows follow
from its last few rows and its first 7 rows.  The sums are small integers,
exact in float32 and float64 alike, so float sums must match bit for bit;
the u32 case (r mod 5, wrapping) checks the integer sum modulo 2^32."""
import numpy as np
import pytest
import torch

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _lengths(rng, n, segs, giant=0):
    """`segs` lengths summing to n: one giant segment (if given), 2 % empty,
    the rest random."""
    w = rng.random(segs)
    w[rng.random(segs) < 0.02] = 0.0
    k = int(rng.integers(0, segs))
    w[k] = 0.0
    rest = n - giant
    ln = np.floor(w / w.sum() * rest).astype(np.int64)
    ln[int(np.argmax(w))] += rest - int(ln.sum())
    ln[k] = giant
    assert ln.sum() == n and (ln >= 0).all()
    return ln


def _device_values(n, feat, m, dtype=torch.float32, chunk=1 << 22):
    v = torch.empty((n, feat) if feat > 1 else (n,), dtype=dtype, device="cuda")
    f = torch.arange(feat, dtype=torch.int64, device="cuda")
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        r = torch.arange(c0, c1, dtype=torch.int64, device="cuda")
        if feat > 1:
            x = (m * r[:, None] + f[None, :]) % 7 - 3
        else:
            x = (m * r) % 7 - 3
        v[c0:c1] = x.to(dtype)
    torch.cuda.synchronize()
    return v


def _expected(off, feat, m):
    """Per (segment, feature): sum, max and its first row, min and its first
    row of ((m r + f) mod 7) - 3 over the segment's rows."""
    lo, hi = off[:-1].astype(object), off[1:].astype(object)
    s = lo.shape[0]
    out = {"sum": np.zeros((s, feat)), "max": np.zeros((s, feat)), "min": np.zeros((s, feat)),
           "argmax": np.full((s, feat), -1, np.int64), "argmin": np.full((s, feat), -1, np.int64)}
    for i in range(s):
        a, b = int(lo[i]), int(hi[i])
        if a == b:
            continue
        for f in range(feat):
            tail = [(m * r + f) % 7 - 3 for r in range(b - (b - a) % 7, b)]
            out["sum"][i, f] = sum(tail)  # full periods of 7 sum to zero
            head = [((m * r + f) % 7 - 3, r) for r in range(a, min(b, a + 7))]
            mx = max(v for v, _ in head)
            mn = min(v for v, _ in head)
            out["max"][i, f], out["argmax"][i, f] = mx, next(r for v, r in head if v == mx)
            out["min"][i, f], out["argmin"][i, f] = mn, next(r for v, r in head if v == mn)
    return out


def _run(vals, off_np, feat, m, ops, what):
    import segmented_reduction_amd as sr
    off = gu.to_gpu(off_np)
    exp = _expected(off_np, feat, m)
    s = off_np.shape[0] - 1
    lens = np.diff(off_np).reshape(s, 1)
    for op in ops:
        gu.say(f"{what} op={op} rows={vals.shape[0]} F={feat} S={s}")
        out, arg = sr.reduce(vals, off, op)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(s, feat)
        if op == "mean":
            want = np.where(lens > 0, exp["sum"] / np.maximum(lens, 1), 0.0).astype(np.float32)
            assert np.allclose(got, want, rtol=0, atol=1e-6), what
            continue
        want = exp[op].astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (what, op)
        if op in ("min", "max"):
            assert np.array_equal(arg.cpu().numpy().reshape(s, feat), exp["arg" + op]), (what, op)
        del out, arg


def test_one_dimensional_past_2_31_rows():
    """2^31 + 2^24 + 5 float32 values (8.7 GB) in 3,000 segments, one of them
    2^31 + 1,000 rows long (its rows cross row 2^31)."""
    rng = np.random.default_rng(31)
    n = 2 ** 31 + 2 ** 24 + 5
    ln = _lengths(rng, n, 3000, giant=2 ** 31 + 1000)
    off = np.zeros(ln.size + 1, dtype=np.int64)
    np.cumsum(ln, out=off[1:])
    vals = _device_values(n, 1, 1)
    _run(vals, off, 1, 1, ("sum", "max", "min", "mean"), "1-D 2^31+")
    _scan_samples(vals, off, rng)
    del vals
    torch.cuda.empty_cache()


def _scan_samples(vals, off, rng):
    """Inclusive segmented sum scan of (r mod 7) - 3, checked at a million
    random rows and at the first and last 64 rows of every segment: the
    value at row r of a segment starting at lo is P(r + 1) - P(lo), with
    P(x) = sum over i < x of (i mod 7) - 3, which depends on x mod 7 only."""
    import segmented_reduction_amd as sr
    n = vals.shape[0]
    gu.say(f"1-D 2^31+ inclusive sum scan rows={n}")
    out = sr.scan(vals, gu.to_gpu(off), "sum")
    torch.cuda.synchronize()
    lo, hi = off[:-1], off[1:]
    nz = hi > lo
    edges = np.concatenate([np.minimum(lo[nz, None] + np.arange(64), hi[nz, None] - 1).ravel(),
                            np.maximum(hi[nz, None] - 1 - np.arange(64), lo[nz, None]).ravel()])
    rows = np.unique(np.concatenate([rng.integers(0, n, 1_000_000), edges, [0, n - 1]]))
    seg = np.searchsorted(off, rows, side="right") - 1  # segment of each row (no row lies past off[-1])
    P = lambda x: (x % 7) * ((x % 7) - 1) // 2 - 3 * (x % 7)
    want = (P(rows + 1) - P(off[seg])).astype(np.float32)
    got = out[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    del out


def test_one_dimensional_u32_sums_wrap_past_2_31_rows():
    rng = np.random.default_rng(32)
    n = 2 ** 31 + 77
    ln = _lengths(rng, n, 500, giant=2 ** 31 - 5)
    off = np.zeros(ln.size + 1, dtype=np.int64)
    np.cumsum(ln, out=off[1:])
    v = torch.empty(n, dtype=torch.int32, device="cuda")
    for c0 in range(0, n, 1 << 26):
        c1 = min(n, c0 + (1 << 26))
        v[c0:c1] = (torch.arange(c0, c1, dtype=torch.int64, device="cuda") % 5 * 1_000_003).to(torch.int32)
    vals = v.view(torch.uint32)
    import segmented_reduction_amd as sr
    gu.say(f"1-D u32 sum rows={n}")
    out, _ = sr.reduce(vals, gu.to_gpu(off), "sum")
    torch.cuda.synchronize()

    def pref(x):  # sum over r < x of (r mod 5) * 1,000,003
        q, rem = divmod(x, 5)
        return (q * 10 + rem * (rem - 1) // 2) * 1_000_003

    want = np.array([(pref(int(off[i + 1])) - pref(int(off[i]))) % 2 ** 32 for i in range(ln.size)], dtype=np.uint64)
    assert np.array_equal(out.cpu().numpy().astype(np.uint64), want)
    del v, vals, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("feat,m,rows", [(64, 1, 21_000_000), (32, 4, 42_000_000), (4, 4, 340_000_000),
                                         (3, 3, 450_000_000), (2, 2, 2_200_000_000)])
def test_rows_past_4_gib(feat, m, rows):
    """5.4 GB of rows of 256 bytes (chunked walk), of 128 bytes (team walk),
    of 16 and 12 bytes (chunks staged through LDS), and 17.6 GB of rows of
    8 bytes: past 2^31 rows."""
    rng = np.random.default_rng(feat)
    ln = _lengths(rng, rows, 300, giant=rows // 3)
    off = np.zeros(ln.size + 1, dtype=np.int64)
    np.cumsum(ln, out=off[1:])
    vals = _device_values(rows, feat, m)
    _run(vals, off, feat, m, ("sum", "max", "min"), f"rows F={feat} past 4 GiB")
    del vals
    torch.cuda.empty_cache()


def test_runs_past_2_31_keys():
    """2^31 + 4,097 keys r // 1000 (runs of 1,000 crossing row 2^31 and every
    tile edge): RLE, unique and start flags against their closed forms."""
    import segmented_reduction_amd as sr
    n = 2 ** 31 + 4097
    runs = (n + 999) // 1000
    keys = torch.empty(n, dtype=torch.int32, device="cuda")
    for c0 in range(0, n, 1 << 26):
        c1 = min(n, c0 + (1 << 26))
        keys[c0:c1] = (torch.arange(c0, c1, dtype=torch.int64, device="cuda") // 1000).to(torch.int32)
    keys = keys.view(torch.uint32)
    want_off = np.minimum(np.arange(runs + 1, dtype=np.int64) * 1000, n)
    gu.say(f"rle n={n}")
    v, ln, off, c = sr.rle(keys)
    assert c == runs
    assert np.array_equal(v.cpu().numpy().astype(np.int64), np.arange(runs))
    assert np.array_equal(ln.cpu().numpy().astype(np.int64), np.diff(want_off))
    assert np.array_equal(off.cpu().numpy(), want_off)
    del v, ln, off
    torch.cuda.empty_cache()
    gu.say(f"unique n={n}")
    uv, uc = sr.unique(keys)
    uc = int(uc.item())
    assert uc == runs and np.array_equal(uv[:uc].cpu().numpy().astype(np.int64), np.arange(runs))
    del uv, keys
    torch.cuda.empty_cache()
    flags = torch.empty(n, dtype=torch.int32, device="cuda")
    for c0 in range(0, n, 1 << 26):
        c1 = min(n, c0 + (1 << 26))
        flags[c0:c1] = ((torch.arange(c0, c1, dtype=torch.int64, device="cuda") % 1000) == 0).to(torch.int32) * 7
    gu.say(f"offsets_from_flags n={n}")
    fo, fc = sr.offsets_from_flags(flags.view(torch.uint32))
    fc = int(fc.item())
    assert fc == runs and np.array_equal(fo[: fc + 1].cpu().numpy(), want_off)
    del flags, fo
    torch.cuda.empty_cache()


@pytest.mark.parametrize("feat,rows", [(4099, 700), (40_000, 90)])
def test_very_wide_rows(feat, rows):
    """Rows of thousands of features: the chunked walk runs over many feature
    blocks and the combine over wide partials (oracle comparison)."""
    import workloads as W
    off, vals = W.ragged(seed=feat, segments=9, mean_len=rows // 10, feat=feat, dtype="f32", empty_frac=0.2,
                         base=3, tail_rows=2, long_segment=rows // 3)
    for op in ("sum", "max"):
        for shares in (None, 7):
            gu.check(vals, off, op, shares=shares, what=f"wide F={feat}")


def test_scratch_beyond_device_memory_is_reported():
    """A call whose scratch cannot be had (2,048 shares x 2^24 features x two
    8-byte partial slots = 512 GiB) returns SEGRED_ERR_OUT_OF_MEMORY before
    any launch, and the next call on the same stream works."""
    import segmented_reduction_amd as sr
    feat = 1 << 24  # the widest row the library accepts
    vals = torch.ones((2, feat), dtype=torch.float32, device="cuda")
    off = torch.tensor([0, 2], dtype=torch.int64, device="cuda")
    gu.say("scratch beyond device memory F=2^24")
    with pytest.raises(sr.SegredError) as e:
        sr.reduce(vals, off, "sum")
    assert e.value.status == 3
    del vals
    torch.cuda.empty_cache()
    small = torch.arange(12, dtype=torch.float32, device="cuda").reshape(3, 4)
    out, _ = sr.reduce(small, torch.tensor([0, 1, 3], dtype=torch.int64, device="cuda"), "sum")
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [[0, 1, 2, 3], [12, 14, 16, 18]]


def test_scatter_and_index_offsets_past_2_31_rows():
    """2^31 + 123 rows scattered by index r mod 1,000,003 (every destination
    gets about 2,147 rows spread over the whole input), values (r mod 7) - 3:
    sums (exact in any order), max with its first row, and the CSR pointer,
    all in closed form."""
    import segmented_reduction_amd as sr
    n, dim = 2 ** 31 + 123, 1_000_003
    c = dim % 7  # 4: step of the residue from one row of a destination to its next
    index = torch.empty(n, dtype=torch.int64, device="cuda")
    vals = torch.empty(n, dtype=torch.float32, device="cuda")
    for c0 in range(0, n, 1 << 26):
        c1 = min(n, c0 + (1 << 26))
        r = torch.arange(c0, c1, dtype=torch.int64, device="cuda")
        index[c0:c1] = r % dim
        vals[c0:c1] = (r % 7 - 3).to(torch.float32)
    del r
    torch.cuda.synchronize()
    d = np.arange(dim, dtype=np.int64)
    K = (n - 1 - d) // dim + 1                      # rows of destination d
    rem = K % 7                                     # full periods of 7 rows sum to zero
    want_sum = np.zeros(dim, dtype=np.int64)
    for j in range(7):
        k = K - rem + j
        want_sum += np.where(j < rem, (d + c * k) % 7 - 3, 0)
    inv = next(x for x in range(1, 7) if (c * x) % 7 == 1)
    k0 = ((6 - d) * inv) % 7                        # first k with residue 6 (value 3); K >= 7 everywhere
    want_arg = d + k0 * dim
    gu.say(f"scatter sum rows={n} dim={dim}")
    out, _ = sr.scatter(vals, index, dim, "sum")
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.int64), want_sum)
    del out
    gu.say(f"scatter max rows={n} dim={dim}")
    out, arg = sr.scatter(vals, index, dim, "max")
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 3.0).all()
    assert np.array_equal(arg.cpu().numpy(), want_arg)
    del out, arg
    gu.say(f"offsets_from_index rows={n} dim={dim}")
    off = sr.offsets_from_index(index, dim)
    torch.cuda.synchronize()
    want_off = np.zeros(dim + 1, dtype=np.int64)
    np.cumsum(K, out=want_off[1:])
    assert np.array_equal(off.cpu().numpy(), want_off)
    del index, vals, off
    torch.cuda.empty_cache()
