"""Segmented reduction over offset-delimited segments on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/segred.h`` (libsegred.so,
built from ``csrc/`` with hipcc).  Every step of the computation runs in the
library's HIP kernels; this module only checks tensors, allocates outputs
with PyTorch and passes device pointers and PyTorch's current HIP stream.
There is no CPU fallback: if the library is missing, calls raise.

    out, arg = reduce(values, offsets, "max")        # values [N] or [N, F] on the GPU
    values, lengths, offsets, count = offsets_from_rle(sorted_keys)
    out, arg = scatter(values, index, dim_size, "max")  # unsorted int64 index [N]
    offsets = offsets_from_index(sorted_index, dim_size)
    prefix = scan(values, offsets, "sum", exclusive=False)  # segmented scan
    pos, word = galloping_search(values, queries, segments)  # lower bounds per segment
    values, count = unique(keys)                       # distinct adjacent values
    offsets, count = offsets_from_flags(start_flags)   # uint32 flags, nonzero = start
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libsegred.so")

SUM, MIN, MAX, MEAN = 0, 1, 2, 3
OPS = {"sum": SUM, "min": MIN, "max": MAX, "mean": MEAN}
DTYPES = {torch.uint32: 0, torch.int32: 1, torch.float32: 2}
STATUS = {0: "SEGRED_OK", 1: "SEGRED_ERR_INVALID_ARGUMENT", 2: "SEGRED_ERR_UNSUPPORTED",
          3: "SEGRED_ERR_OUT_OF_MEMORY", 4: "SEGRED_ERR_HIP", 5: "SEGRED_ERR_SCRATCH_LIMIT"}


class SegredError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


_lock = threading.Lock()
_lib = None


def library(path: str | None = None):
    """Load libsegred.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            p = path or LIB_PATH
            if not os.path.exists(p):
                raise RuntimeError(f"libsegred.so not found at {p}; build it with "
                                   "`python -m segmented_reduction_amd.build_lib`")
            lib = ctypes.CDLL(p)
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            lib.segred_reduce.argtypes = [vp, i32, i64, vp, i64, i32, vp, vp, vp]
            lib.segred_reduce.restype = ctypes.c_int
            lib.segred_reduce_noalloc.argtypes = [vp, i32, i64, vp, i64, i32, vp, vp, vp]
            lib.segred_reduce_noalloc.restype = ctypes.c_int
            lib.segred_reduce_device_count.argtypes = [vp, i32, i64, vp, vp, i64, i32, vp, vp, vp]
            lib.segred_reduce_device_count.restype = ctypes.c_int
            lib.segred_offsets_from_rle.argtypes = [vp, i64, vp, vp, vp, vp, vp]
            lib.segred_offsets_from_rle.restype = ctypes.c_int
            lib.segred_scatter_reduce.argtypes = [vp, i32, i64, i64, vp, i64, i32, vp, vp, vp]
            lib.segred_scatter_reduce.restype = ctypes.c_int
            lib.segred_offsets_from_index.argtypes = [vp, i64, i64, vp, vp]
            lib.segred_offsets_from_index.restype = ctypes.c_int
            lib.segred_scan.argtypes = [vp, i32, i64, vp, i64, i32, i32, vp, vp]
            lib.segred_scan.restype = ctypes.c_int
            lib.segred_galloping_search.argtypes = [vp, i32, i64, i64, vp, i64, vp, i64, vp, i64, i64, i32, vp,
                                                    vp, i32, vp]
            lib.segred_galloping_search.restype = ctypes.c_int
            lib.segred_unique.argtypes = [vp, i64, vp, vp, vp]
            lib.segred_unique.restype = ctypes.c_int
            lib.segred_offsets_from_flags.argtypes = [vp, i64, vp, vp, vp]
            lib.segred_offsets_from_flags.restype = ctypes.c_int
            lib.segred_status_string.argtypes = [ctypes.c_int]
            lib.segred_status_string.restype = ctypes.c_char_p
            lib.segred_set_shares.argtypes = [i64]
            lib.segred_set_shares.restype = ctypes.c_int
            lib.segred_get_shares.argtypes = [i32, i32, i64]
            lib.segred_get_shares.restype = i64
            lib.segred_resident_waves.argtypes = [i32, i32, i64]
            lib.segred_resident_waves.restype = i64
            lib.segred_timing_enable.argtypes = [ctypes.c_int]
            lib.segred_timing_enable.restype = ctypes.c_int
            lib.segred_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64),
                                              ctypes.POINTER(ctypes.c_float), i64]
            lib.segred_timing_read.restype = ctypes.c_int
            lib.segred_probe_stream.argtypes = [vp, i64, vp, i32, vp, i32, vp]
            lib.segred_probe_stream.restype = ctypes.c_int
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().segred_status_string(int(status)).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise SegredError(rc, what)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def reduce(values: torch.Tensor, offsets: torch.Tensor, op: str, *, want_arg: bool = True,
           out: torch.Tensor | None = None, arg: torch.Tensor | None = None,
           num_segments: torch.Tensor | None = None):
    """Segmented ``op`` ("sum", "min", "max", "mean") of ``values`` over ``offsets``.

    values  [N] or [N, ...] uint32 / int32 / float32 on a GPU, contiguous;
            trailing dimensions are flattened into F features per row.
    offsets int64 [S + 1] on the same GPU; segment s is rows offsets[s]..offsets[s+1]-1.
    num_segments  optional one-element int64 GPU tensor: the segment count is
            then read on the device (segred_reduce_device_count); offsets
            and the outputs are its capacity and rows past the count are
            left as they were.
    Returns (out [S, ...], arg [S, ...] int64 or None).  arg is the row of
    the extremum for min/max (lowest on ties, -1 for empty segments).
    """
    if op not in OPS:
        raise ValueError(f"op must be one of {sorted(OPS)}")
    if not (values.is_cuda and offsets.is_cuda):
        raise ValueError("values and offsets must be GPU tensors")
    if values.dtype not in DTYPES:
        raise TypeError(f"values dtype {values.dtype} is not uint32, int32 or float32")
    if offsets.dtype != torch.int64 or offsets.dim() != 1 or offsets.numel() < 1:
        raise ValueError("offsets must be a 1-D int64 tensor with S + 1 entries")
    if values.device != offsets.device:
        raise ValueError("values and offsets must be on the same device")
    if not values.is_contiguous() or not offsets.is_contiguous():
        raise ValueError("values and offsets must be contiguous")
    if values.dim() == 0:
        raise ValueError("values needs at least one dimension")
    s = offsets.numel() - 1
    feat_shape = tuple(values.shape[1:])
    feat = 1
    for d in feat_shape:
        feat *= d
    if feat < 1:
        raise ValueError("values has an empty feature dimension")
    odt = torch.float32 if op == "mean" else values.dtype
    if out is None:
        out = torch.empty((s,) + feat_shape, dtype=odt, device=values.device)
    want = op in ("min", "max") and want_arg
    if want and arg is None:
        arg = torch.empty((s,) + feat_shape, dtype=torch.int64, device=values.device)
    if not want:
        arg = None
    if num_segments is not None:
        if (not num_segments.is_cuda or num_segments.dtype != torch.int64 or num_segments.numel() != 1
                or num_segments.device != values.device):
            raise ValueError("num_segments must be a one-element int64 tensor on the values' device")
        with torch.cuda.device(values.device):
            rc = library().segred_reduce_device_count(
                values.data_ptr(), DTYPES[values.dtype], feat, offsets.data_ptr(), num_segments.data_ptr(), s,
                OPS[op], out.data_ptr(), arg.data_ptr() if arg is not None else None, _stream(values.device))
        _check(rc, "segred_reduce_device_count")
        return out, arg
    with torch.cuda.device(values.device):
        rc = library().segred_reduce(values.data_ptr(), DTYPES[values.dtype], feat, offsets.data_ptr(), s,
                                     OPS[op], out.data_ptr(), arg.data_ptr() if arg is not None else None,
                                     _stream(values.device))
    _check(rc, "segred_reduce")
    return out, arg


def offsets_from_rle(keys: torch.Tensor):
    """Run-length encode uint32 ``keys`` (adjacent runs) on the GPU.

    Returns (values [n], lengths [n], offsets [n + 1], count [1] int64), all on
    the GPU and written asynchronously; only values[:count], lengths[:count]
    and offsets[:count + 1] are meaningful.
    """
    if not keys.is_cuda or keys.dtype != torch.uint32 or keys.dim() != 1 or not keys.is_contiguous():
        raise ValueError("keys must be a contiguous 1-D uint32 GPU tensor")
    n = keys.numel()
    dev = keys.device
    values = torch.empty(max(n, 1), dtype=torch.uint32, device=dev)
    lengths = torch.empty(max(n, 1), dtype=torch.uint32, device=dev)
    offsets = torch.empty(n + 1, dtype=torch.int64, device=dev)
    count = torch.empty(1, dtype=torch.int64, device=dev)
    with torch.cuda.device(dev):
        rc = library().segred_offsets_from_rle(keys.data_ptr() if n else None, n, values.data_ptr(),
                                               lengths.data_ptr(), offsets.data_ptr(), count.data_ptr(),
                                               _stream(dev))
    _check(rc, "segred_offsets_from_rle")
    return values, lengths, offsets, count


def rle(keys: torch.Tensor):
    """``offsets_from_rle`` followed by the one 8-byte readback of the count:
    returns (values[:count], lengths[:count], offsets[:count + 1], count)."""
    values, lengths, offsets, count = offsets_from_rle(keys)
    c = int(count.item())
    return values[:c], lengths[:c], offsets[: c + 1], c


def scatter(values: torch.Tensor, index: torch.Tensor, dim_size: int, op: str, *, want_arg: bool = True,
            out: torch.Tensor | None = None, arg: torch.Tensor | None = None):
    """Scatter ``op`` ("sum", "min", "max", "mean"): row r of ``values`` goes
    to output ``index[r]`` (segred_scatter_reduce).

    values  [N] or [N, ...] uint32 / int32 / float32 on a GPU, contiguous.
    index   int64 [N] on the same GPU, any order; entries outside
            [0, dim_size) are ignored.
    Returns (out [dim_size, ...], arg [dim_size, ...] int64 or None).  Float
    sums use atomic additions and may differ in the last bits run to run.
    """
    if op not in OPS:
        raise ValueError(f"op must be one of {sorted(OPS)}")
    if not (values.is_cuda and index.is_cuda) or values.device != index.device:
        raise ValueError("values and index must be tensors on the same GPU")
    if values.dtype not in DTYPES:
        raise TypeError(f"values dtype {values.dtype} is not uint32, int32 or float32")
    if values.dim() == 0 or not values.is_contiguous():
        raise ValueError("values must be contiguous with at least one dimension")
    if index.dtype != torch.int64 or index.dim() != 1 or not index.is_contiguous():
        raise ValueError("index must be a contiguous 1-D int64 tensor")
    n = values.shape[0]
    if index.numel() != n:
        raise ValueError("index needs one entry per row of values")
    dim_size = int(dim_size)
    if dim_size < 0:
        raise ValueError("dim_size must be >= 0")
    feat_shape = tuple(values.shape[1:])
    feat = 1
    for d in feat_shape:
        feat *= d
    if feat < 1:
        raise ValueError("values has an empty feature dimension")
    odt = torch.float32 if op == "mean" else values.dtype
    if out is None:
        out = torch.empty((dim_size,) + feat_shape, dtype=odt, device=values.device)
    want = op in ("min", "max") and want_arg
    if want and arg is None:
        arg = torch.empty((dim_size,) + feat_shape, dtype=torch.int64, device=values.device)
    if not want:
        arg = None
    with torch.cuda.device(values.device):
        rc = library().segred_scatter_reduce(values.data_ptr() if n else None, DTYPES[values.dtype], feat, n,
                                             index.data_ptr() if n else None, dim_size, OPS[op],
                                             out.data_ptr() if dim_size else None,
                                             arg.data_ptr() if (arg is not None and dim_size) else None,
                                             _stream(values.device))
    _check(rc, "segred_scatter_reduce")
    return out, arg


def offsets_from_index(index: torch.Tensor, dim_size: int) -> torch.Tensor:
    """CSR offsets [dim_size + 1] of an int64 GPU ``index``: offsets[s] = rows
    with index in [0, s) (segred_offsets_from_index)."""
    if not index.is_cuda or index.dtype != torch.int64 or index.dim() != 1 or not index.is_contiguous():
        raise ValueError("index must be a contiguous 1-D int64 GPU tensor")
    dim_size = int(dim_size)
    if dim_size < 0:
        raise ValueError("dim_size must be >= 0")
    n = index.numel()
    offsets = torch.empty(dim_size + 1, dtype=torch.int64, device=index.device)
    with torch.cuda.device(index.device):
        rc = library().segred_offsets_from_index(index.data_ptr() if n else None, n, dim_size,
                                                 offsets.data_ptr(), _stream(index.device))
    _check(rc, "segred_offsets_from_index")
    return offsets


def scan(values: torch.Tensor, offsets: torch.Tensor, op: str, *, exclusive: bool = False,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """Segmented inclusive / exclusive ``op`` ("sum", "min", "max") scan of
    ``values`` over ``offsets`` (segred_scan).

    Returns ``out`` with the shape and dtype of ``values``; rows outside
    [offsets[0], offsets[-1]) are left as they were in ``out`` (uninitialised
    when ``out`` is not given)."""
    if op not in ("sum", "min", "max"):
        raise ValueError("op must be one of ['max', 'min', 'sum']")
    if not (values.is_cuda and offsets.is_cuda) or values.device != offsets.device:
        raise ValueError("values and offsets must be tensors on the same GPU")
    if values.dtype not in DTYPES:
        raise TypeError(f"values dtype {values.dtype} is not uint32, int32 or float32")
    if offsets.dtype != torch.int64 or offsets.dim() != 1 or offsets.numel() < 1:
        raise ValueError("offsets must be a 1-D int64 tensor with S + 1 entries")
    if values.dim() == 0 or not values.is_contiguous() or not offsets.is_contiguous():
        raise ValueError("values and offsets must be contiguous; values needs a row dimension")
    feat = 1
    for d in values.shape[1:]:
        feat *= d
    if feat < 1:
        raise ValueError("values has an empty feature dimension")
    if out is None:
        out = torch.empty_like(values)
    elif out.shape != values.shape or out.dtype != values.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous with the shape and dtype of values")
    s = offsets.numel() - 1
    with torch.cuda.device(values.device):
        rc = library().segred_scan(values.data_ptr(), DTYPES[values.dtype], feat, offsets.data_ptr(), s, OPS[op],
                                   int(bool(exclusive)), out.data_ptr(), _stream(values.device))
    _check(rc, "segred_scan")
    return out


def galloping_search(values: torch.Tensor, queries: torch.Tensor, segments: torch.Tensor, *,
                     value_order: torch.Tensor | None = None, value_stride: int = 1, value_count: int | None = None,
                     max_query_count: int | None = None, queries_per_tile: int = 32,
                     out: torch.Tensor | None = None, validation: torch.Tensor | None = None,
                     preserve_validation: bool = False):
    """Lower bounds of ``queries`` over segmented sorted ``values``
    (segred_galloping_search).  ``values`` and ``queries`` are uint32 or
    float32 GPU tensors of one dtype; ``segments`` int64 [S, 4] records
    (vo, vc, qo, qc) on the GPU.  ``max_query_count`` defaults to the
    queries' length (no host read of the records).  Returns (out int64
    [len(queries)], validation uint32 [1]), both on the GPU."""
    if values.dtype not in (torch.uint32, torch.float32) or queries.dtype != values.dtype:
        raise TypeError("values and queries must both be uint32 or both float32")
    for t in (values, queries, segments):
        if not t.is_cuda or t.device != values.device or not t.is_contiguous():
            raise ValueError("values, queries and segments must be contiguous tensors on one GPU")
    if segments.dtype != torch.int64 or segments.dim() != 2 or segments.shape[1] != 4:
        raise ValueError("segments must be an int64 [S, 4] tensor")
    if value_order is not None and (value_order.dtype != torch.uint32 or not value_order.is_cuda
                                    or value_order.device != values.device or not value_order.is_contiguous()):
        raise ValueError("value_order must be a contiguous uint32 tensor on the values' GPU")
    n = values.numel()
    vcount = value_count if value_count is not None else (n + value_stride - 1) // value_stride
    qn = queries.numel()
    mq = qn if max_query_count is None else int(max_query_count)
    dev = values.device
    if out is None:
        out = torch.empty(qn, dtype=torch.int64, device=dev)
    if validation is None:
        validation = torch.zeros(1, dtype=torch.int32, device=dev).view(torch.uint32)
    with torch.cuda.device(dev):
        rc = library().segred_galloping_search(
            values.data_ptr() if n else None, DTYPES[values.dtype], vcount, value_stride,
            value_order.data_ptr() if value_order is not None else None,
            value_order.numel() if value_order is not None else 0,
            queries.data_ptr() if qn else None, qn, segments.data_ptr() if segments.numel() else None,
            segments.shape[0], mq, queries_per_tile, out.data_ptr() if qn else None, validation.data_ptr(),
            int(bool(preserve_validation)), _stream(dev))
    _check(rc, "segred_galloping_search")
    return out, validation


def unique(keys: torch.Tensor):
    """Distinct adjacent values of uint32 ``keys`` (segred_unique).

    Returns (values [n], count [1] int64) on the GPU, written asynchronously;
    only values[:count] is meaningful."""
    if not keys.is_cuda or keys.dtype != torch.uint32 or keys.dim() != 1 or not keys.is_contiguous():
        raise ValueError("keys must be a contiguous 1-D uint32 GPU tensor")
    n = keys.numel()
    values = torch.empty(max(n, 1), dtype=torch.uint32, device=keys.device)
    count = torch.empty(1, dtype=torch.int64, device=keys.device)
    with torch.cuda.device(keys.device):
        rc = library().segred_unique(keys.data_ptr() if n else None, n, values.data_ptr(), count.data_ptr(),
                                     _stream(keys.device))
    _check(rc, "segred_unique")
    return values, count


def offsets_from_flags(flags: torch.Tensor):
    """Offsets of the segments that uint32 start ``flags`` open (nonzero =
    start; segred_offsets_from_flags).

    Returns (offsets [n + 1], count [1] int64) on the GPU, written
    asynchronously; only offsets[:count + 1] is meaningful."""
    if not flags.is_cuda or flags.dtype != torch.uint32 or flags.dim() != 1 or not flags.is_contiguous():
        raise ValueError("flags must be a contiguous 1-D uint32 GPU tensor")
    n = flags.numel()
    offsets = torch.empty(n + 1, dtype=torch.int64, device=flags.device)
    count = torch.empty(1, dtype=torch.int64, device=flags.device)
    with torch.cuda.device(flags.device):
        rc = library().segred_offsets_from_flags(flags.data_ptr() if n else None, n, offsets.data_ptr(),
                                                 count.data_ptr(), _stream(flags.device))
    _check(rc, "segred_offsets_from_flags")
    return offsets, count


def set_shares(shares: int):
    """Override the work partition (0 = default); see segred_set_shares."""
    _check(library().segred_set_shares(int(shares)), "segred_set_shares")


def get_shares(dtype=torch.float32, op: str = "sum", feat: int = 1) -> int:
    return int(library().segred_get_shares(DTYPES[dtype], OPS[op], int(feat)))


def timing_enable(enable: bool = True):
    _check(library().segred_timing_enable(1 if enable else 0), "segred_timing_enable")


def timing_read(capacity: int = 8192):
    """(total ms, launches, per-launch ms list) of the streaming kernels since the last read:
    each is the kernel's own stop event minus its own start event."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    each = (ctypes.c_float * max(capacity, 1))()
    _check(library().segred_timing_read(ctypes.byref(ms), ctypes.byref(n), each, capacity), "segred_timing_read")
    return ms.value, n.value, [each[i] for i in range(min(n.value, capacity))]


def probe_stream(src: torch.Tensor, write_every: int = 0, waves: int = 4096,
                 dst: torch.Tensor | None = None):
    """Streaming-rate probe (measurement context, see segred_probe_stream).

    src  contiguous float32 GPU tensor whose size in bytes is a multiple of
         1,024, read once by `waves` waves over contiguous shares.
    write_every  0 (read only) or 1..1024: one 1 KB block is written per
         `write_every` blocks read, to `dst` (float32, at least
         floor(blocks / write_every) * 256 elements; allocated when None).
    Returns (wave_sums [waves] float32, dst or None).
    """
    if not src.is_cuda or src.dtype != torch.float32 or not src.is_contiguous():
        raise ValueError("src must be a contiguous float32 GPU tensor")
    nbytes = src.numel() * 4
    if write_every > 0 and dst is None:
        dst = torch.empty((nbytes // 1024 // write_every) * 256, dtype=torch.float32, device=src.device)
    if dst is not None and (not dst.is_cuda or dst.dtype != torch.float32 or not dst.is_contiguous()
                            or dst.device != src.device):
        raise ValueError("dst must be a contiguous float32 tensor on the device of src")
    if write_every > 0 and dst.numel() < (nbytes // 1024 // write_every) * 256:
        raise ValueError("dst is smaller than one 1 KB block per write_every blocks of src")
    sums = torch.empty(max(int(waves), 1), dtype=torch.float32, device=src.device)
    _check(library().segred_probe_stream(
        ctypes.c_void_p(src.data_ptr()), nbytes,
        ctypes.c_void_p(dst.data_ptr() if dst is not None and write_every > 0 else 0),
        int(write_every), ctypes.c_void_p(sums.data_ptr()), int(waves),
        ctypes.c_void_p(_stream(src.device))), "segred_probe_stream")
    return sums, (dst if write_every > 0 else None)
