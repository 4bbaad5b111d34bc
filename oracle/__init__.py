"""CPU oracle for segmented reduction, run-length encoding and scatter reduction.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product (the HIP library
and its Python binding) never does.  It shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, one thread, double-precision
accumulation, rows in ascending order); this module builds it with gcc and
marshals numpy arrays into it.  See the header of ``oracle.c`` for the pages
and readings each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"u32": 0, "i32": 1, "f32": 2}
OPS = {"sum": 0, "min": 1, "max": 2, "mean": 3}
_NP = {"u32": np.uint32, "i32": np.int32, "f32": np.float32}

_lock = threading.Lock()
_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str | None = None):
    """Load a compiled oracle library (building the default one if absent)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.oracle_reduce.argtypes = [vp, i32, i64, vp, i64, i32, vp, vp, vp, vp]
    lib.oracle_reduce.restype = ctypes.c_int
    lib.oracle_rle.argtypes = [vp, i64, vp, vp, vp, vp]
    lib.oracle_rle.restype = ctypes.c_int
    lib.oracle_scatter.argtypes = [vp, i32, i64, i64, vp, i64, i32, vp, vp, vp, vp]
    lib.oracle_scatter.restype = ctypes.c_int
    lib.oracle_offsets_from_index.argtypes = [vp, i64, i64, vp]
    lib.oracle_offsets_from_index.restype = ctypes.c_int
    lib.oracle_scan.argtypes = [vp, i32, i64, vp, i64, i32, i32, vp, vp, vp]
    lib.oracle_scan.restype = ctypes.c_int
    lib.oracle_lower_bounds.argtypes = [vp, i32, i64, i64, vp, i64, vp, i64, vp, i64, i64, i64, vp, vp, i32]
    lib.oracle_lower_bounds.restype = ctypes.c_int
    lib.oracle_unique.argtypes = [vp, i64, vp, vp]
    lib.oracle_unique.restype = ctypes.c_int
    lib.oracle_offsets_from_flags.argtypes = [vp, i64, vp, vp]
    lib.oracle_offsets_from_flags.restype = ctypes.c_int
    lib.oracle_order_key.argtypes = [ctypes.c_uint32, i32]
    lib.oracle_order_key.restype = ctypes.c_uint32
    return lib


def dtype_name(arr: np.ndarray) -> str:
    for name, t in _NP.items():
        if arr.dtype == t:
            return name
    raise TypeError(f"unsupported dtype {arr.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


class Reduced:
    """Result of ``reduce``: out [S, F]; arg [S, F] (min/max);
    ref and mag [S, F] float64 (float32 sum/mean: the double result and sum|x|)."""

    def __init__(self, out, arg=None, ref=None, mag=None):
        self.out, self.arg, self.ref, self.mag = out, arg, ref, mag


def segment_ranges(offsets: np.ndarray, parts: int):
    """Split segments [0, S) into ``parts`` contiguous ranges of about equal
    row counts (used to run the oracle on several host threads; each segment
    is still reduced by one sequential pass, so results do not depend on the
    split)."""
    s = int(offsets.shape[0]) - 1
    o0, o1 = int(offsets[0]), int(offsets[-1])
    cuts = [0]
    for k in range(1, parts):
        r = o0 + (o1 - o0) * k // parts
        cuts.append(min(s, max(cuts[-1], int(np.searchsorted(offsets, r, side="left")))))
    cuts.append(s)
    return [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def reduce(values: np.ndarray, offsets: np.ndarray, op: str, lib=None, threads: int = 1) -> Reduced:
    """Segmented reduction of ``values`` ([rows] or [rows, F]) over int64 ``offsets``.

    ``threads`` > 1 runs the same C function on that many host threads, each
    over a contiguous range of segments (segment_ranges); every segment is
    computed exactly as with one thread."""
    lib = lib or load()
    values = np.ascontiguousarray(values)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    dt = dtype_name(values)
    feat = 1 if values.ndim == 1 else int(np.prod(values.shape[1:]))
    s = int(offsets.shape[0]) - 1
    if s < 0:
        raise ValueError("offsets needs at least one entry")
    out = np.zeros((s, feat), dtype=np.float32 if op == "mean" else _NP[dt])
    arg = np.zeros((s, feat), dtype=np.int64) if op in ("min", "max") else None
    ref = mag = None
    if dt == "f32" and op in ("sum", "mean"):
        ref = np.zeros((s, feat), dtype=np.float64)
        mag = np.zeros((s, feat), dtype=np.float64)
    def run(a, b):
        def at(x, row):
            return None if x is None else x.ctypes.data + row * x.strides[0]
        return lib.oracle_reduce(_ptr(values), DTYPES[dt], feat, offsets.ctypes.data + a * 8, b - a, OPS[op],
                                 at(out, a), at(arg, a), at(ref, a), at(mag, a))

    if threads <= 1 or s < 2:
        rcs = [run(0, s)]
    else:
        from concurrent.futures import ThreadPoolExecutor
        ranges = segment_ranges(offsets, threads)
        with ThreadPoolExecutor(max_workers=len(ranges)) as pool:
            rcs = list(pool.map(lambda ab: run(*ab), ranges))
    if any(rc != 0 for rc in rcs):
        raise ValueError(f"oracle_reduce rejected dtype={dt} op={op} feat={feat}")
    return Reduced(out, arg, ref, mag)


def rle(keys: np.ndarray, lib=None):
    """Run-length encode uint32 ``keys``: returns (values, lengths, offsets, count),
    each array trimmed to its valid prefix (offsets has count + 1 entries)."""
    lib = lib or load()
    keys = np.ascontiguousarray(keys, dtype=np.uint32)
    n = int(keys.shape[0])
    values = np.zeros(max(n, 1), dtype=np.uint32)
    lengths = np.zeros(max(n, 1), dtype=np.uint32)
    offsets = np.zeros(n + 1, dtype=np.int64)
    count = np.zeros(1, dtype=np.int64)
    rc = lib.oracle_rle(_ptr(keys), n, _ptr(values), _ptr(lengths), _ptr(offsets), _ptr(count))
    if rc != 0:
        raise ValueError("oracle_rle rejected its input")
    c = int(count[0])
    return values[:c], lengths[:c], offsets[: c + 1], c


class Scanned:
    """Result of a segmented scan: ``out`` [rows, F] (rows outside the
    segments hold ``fill``), ``ref``/``mag`` float64 prefixes of x and |x|
    for float32 sums (else None)."""

    def __init__(self, out, ref, mag):
        self.out, self.ref, self.mag = out, ref, mag


def scan(values: np.ndarray, offsets: np.ndarray, op: str, exclusive: bool = False, fill=0, lib=None) -> Scanned:
    """Segmented inclusive / exclusive scan (op in sum, min, max) of
    ``values`` ([rows] or [rows, F]) over int64 ``offsets`` [S + 1]."""
    lib = lib or load()
    values = np.ascontiguousarray(values)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    dt = dtype_name(values)
    feat = 1 if values.ndim == 1 else int(np.prod(values.shape[1:]))
    rows = int(values.shape[0])
    out = np.full((rows, feat), fill, dtype=_NP[dt])
    ref = mag = None
    if dt == "f32" and op == "sum":
        ref = np.zeros((rows, feat), dtype=np.float64)
        mag = np.zeros((rows, feat), dtype=np.float64)
    rc = lib.oracle_scan(_ptr(values), DTYPES[dt], feat, _ptr(offsets), int(offsets.shape[0]) - 1, OPS[op],
                         int(bool(exclusive)), _ptr(out), _ptr(ref), _ptr(mag))
    if rc != 0:
        raise ValueError(f"oracle_scan rejected dtype={dt} op={op} feat={feat} (rc={rc})")
    return Scanned(out, ref, mag)


def lower_bounds(values: np.ndarray, queries: np.ndarray, segments: np.ndarray, *, stride: int = 1,
                 order: np.ndarray | None = None, max_qc: int | None = None, tile: int = 32,
                 out: np.ndarray | None = None, validation: int = 0, preserve: bool = False,
                 value_count: int | None = None, lib=None):
    """Lower bounds of ``queries`` over segmented sorted ``values`` (uint32 or
    float32, same dtype); ``segments`` int64 [S, 4] of (vo, vc, qo, qc).
    Returns (out int64 [len(queries)], validation word)."""
    lib = lib or load()
    values = np.ascontiguousarray(values)
    queries = np.ascontiguousarray(queries, dtype=values.dtype)
    segments = np.ascontiguousarray(segments, dtype=np.int64).reshape(-1, 4)
    dt = dtype_name(values)
    if out is None:
        out = np.full(queries.shape[0], -7, dtype=np.int64)
    out = np.ascontiguousarray(out, dtype=np.int64)
    word = np.array([validation], dtype=np.uint32)
    if order is not None:
        order = np.ascontiguousarray(order, dtype=np.uint32)
    if max_qc is None:
        max_qc = int(segments[:, 3].max()) if segments.shape[0] else 0
    if value_count is None:
        value_count = (values.shape[0] + stride - 1) // stride
    rc = lib.oracle_lower_bounds(_ptr(values), DTYPES[dt], int(value_count), stride, _ptr(order), 0 if order is None else order.shape[0], _ptr(queries),
                                 queries.shape[0], _ptr(segments), segments.shape[0], int(max_qc), int(tile),
                                 _ptr(out), _ptr(word), int(bool(preserve)))
    if rc != 0:
        raise ValueError(f"oracle_lower_bounds rejected its arguments (rc={rc})")
    return out, int(word[0])


def unique(keys: np.ndarray, lib=None):
    """Distinct adjacent values of uint32 ``keys``: returns (values[:count], count)."""
    lib = lib or load()
    keys = np.ascontiguousarray(keys, dtype=np.uint32)
    n = int(keys.shape[0])
    values = np.zeros(max(n, 1), dtype=np.uint32)
    count = np.zeros(1, dtype=np.int64)
    if lib.oracle_unique(_ptr(keys), n, _ptr(values), _ptr(count)) != 0:
        raise ValueError("oracle_unique rejected its input")
    c = int(count[0])
    return values[:c], c


def offsets_from_flags(flags: np.ndarray, lib=None):
    """Offsets of the segments that uint32 start ``flags`` (nonzero = start)
    open: returns (offsets[:count + 1], count)."""
    lib = lib or load()
    flags = np.ascontiguousarray(flags, dtype=np.uint32)
    n = int(flags.shape[0])
    offsets = np.zeros(n + 1, dtype=np.int64)
    count = np.zeros(1, dtype=np.int64)
    if lib.oracle_offsets_from_flags(_ptr(flags), n, _ptr(offsets), _ptr(count)) != 0:
        raise ValueError("oracle_offsets_from_flags rejected its input")
    c = int(count[0])
    return offsets[: c + 1], c


def order_key(bits: int, dtype: str, lib=None) -> int:
    """The monotone uint32 key the oracle orders min/max by."""
    lib = lib or load()
    return int(lib.oracle_order_key(ctypes.c_uint32(bits & 0xFFFFFFFF), DTYPES[dtype]))


def scatter(values: np.ndarray, index: np.ndarray, dim_size: int, op: str, lib=None) -> Reduced:
    """Scatter reduction: row r of ``values`` ([rows] or [rows, F]) goes to
    output ``index[r]`` (int64, any order; rows outside [0, dim_size) are
    ignored).  Returns a ``Reduced`` with dim_size outputs."""
    lib = lib or load()
    values = np.ascontiguousarray(values)
    index = np.ascontiguousarray(index, dtype=np.int64)
    dt = dtype_name(values)
    feat = 1 if values.ndim == 1 else int(np.prod(values.shape[1:]))
    rows = int(values.shape[0])
    if index.shape[0] != rows:
        raise ValueError("index needs one entry per row")
    out = np.zeros((dim_size, feat), dtype=np.float32 if op == "mean" else _NP[dt])
    arg = np.zeros((dim_size, feat), dtype=np.int64) if op in ("min", "max") else None
    ref = mag = None
    if dt == "f32" and op in ("sum", "mean"):
        ref = np.zeros((dim_size, feat), dtype=np.float64)
        mag = np.zeros((dim_size, feat), dtype=np.float64)
    rc = lib.oracle_scatter(_ptr(values), DTYPES[dt], feat, rows, _ptr(index), int(dim_size), OPS[op],
                            _ptr(out), _ptr(arg), _ptr(ref), _ptr(mag))
    if rc != 0:
        raise ValueError(f"oracle_scatter rejected dtype={dt} op={op} feat={feat} (rc={rc})")
    return Reduced(out, arg, ref, mag)


def offsets_from_index(index: np.ndarray, dim_size: int, lib=None) -> np.ndarray:
    """CSR offsets [dim_size + 1] of an int64 index (rows outside the range not counted)."""
    lib = lib or load()
    index = np.ascontiguousarray(index, dtype=np.int64)
    offsets = np.zeros(int(dim_size) + 1, dtype=np.int64)
    rc = lib.oracle_offsets_from_index(_ptr(index), int(index.shape[0]), int(dim_size), _ptr(offsets))
    if rc != 0:
        raise ValueError("oracle_offsets_from_index rejected its input")
    return offsets
