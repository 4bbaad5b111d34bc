"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before any device work."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "segred.h")
INSTRUMENT = os.path.join(ROOT, "include", "segred_instrument.h")
CSRC = os.path.join(ROOT, "segmented_reduction_amd", "csrc")


def _lib():
    import segmented_reduction_amd as sr
    if not os.path.exists(sr.LIB_PATH):
        from segmented_reduction_amd import build_lib
        build_lib.build()
    return sr.library()


def _declared(path=HEADER):
    text = open(path).read()
    return sorted(set(re.findall(r"\b(segred_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("segred_reduce", "segred_offsets_from_rle", "segred_status_string", "segred_scatter_reduce",
                     "segred_offsets_from_index", "segred_unique", "segred_offsets_from_flags", "segred_scan",
                     "segred_galloping_search"):
        assert required in names


def test_public_header_holds_only_the_method():
    """Test and benchmark hooks live in their own header, not in the ABI."""
    names = _declared()
    for hook in _declared(INSTRUMENT):
        assert hook not in names, hook
    assert set(_declared(INSTRUMENT)) == {"segred_set_shares", "segred_get_shares", "segred_resident_waves",
                                          "segred_timing_enable", "segred_timing_read", "segred_probe_stream"}


def test_library_exports_every_declared_symbol():
    lib = _lib()
    import segmented_reduction_amd as sr
    out = subprocess.run(["nm", "-D", "--defined-only", sr.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (segred_\w+)", out.stdout))
    for name in _declared() + _declared(INSTRUMENT):
        assert name in exported, name
        assert hasattr(lib, name), name


def test_status_strings():
    lib = _lib()
    for code in range(5):
        assert lib.segred_status_string(code)
    assert lib.segred_status_string(99) == b"unknown status"


FAKE = 0x10000  # a non-null, aligned host value; never dereferenced (rejected or S == 0)


@pytest.mark.parametrize("args,expect", [
    # (values, dtype, feat, offsets, S, op, out, arg) -> status
    ((FAKE, 2, 1, FAKE, -1, 0, FAKE, None), 1),        # S < 0
    ((FAKE, 2, 0, FAKE, 4, 0, FAKE, None), 1),         # feat < 1
    ((FAKE, 3, 1, FAKE, 4, 0, FAKE, None), 1),         # dtype out of range
    ((FAKE, -1, 1, FAKE, 4, 0, FAKE, None), 1),
    ((FAKE, 2, 1, FAKE, 4, 4, FAKE, None), 1),         # op out of range
    ((FAKE, 0, 1, FAKE, 4, 3, FAKE, None), 2),         # MEAN of u32
    ((FAKE, 1, 1, FAKE, 4, 3, FAKE, None), 2),         # MEAN of i32
    ((FAKE, 2, 2 ** 24 + 1, FAKE, 4, 0, FAKE, None), 2),  # more features than the 32-bit chunk offsets allow
    ((None, 2, 1, FAKE, 4, 0, FAKE, None), 1),         # null values
    ((FAKE, 2, 1, None, 4, 0, FAKE, None), 1),         # null offsets
    ((FAKE, 2, 1, FAKE, 4, 0, None, None), 1),         # null out
    ((FAKE + 2, 2, 1, FAKE, 4, 0, FAKE, None), 1),     # values not 4-byte aligned
    ((FAKE, 2, 1, FAKE + 4, 4, 0, FAKE, None), 1),     # offsets not 8-byte aligned
    ((FAKE, 2, 1, FAKE, 4, 0, FAKE + 1, None), 1),     # out not 4-byte aligned
    ((FAKE, 2, 1, FAKE, 4, 1, FAKE, FAKE + 4), 1),     # arg not 8-byte aligned
    ((None, 2, 1, None, 0, 0, None, None), 0),         # S == 0 enqueues nothing
    ((FAKE, 2, 7, FAKE, 0, 2, FAKE, None), 0),
])
def test_reduce_argument_checks(args, expect):
    lib = _lib()
    assert lib.segred_reduce(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    # (values, dtype, feat, offsets, count_dev, max_S, op, out, arg) -> status
    ((FAKE, 2, 1, FAKE, None, 4, 0, FAKE, None), 1),   # null device count
    ((FAKE, 2, 1, FAKE, FAKE + 4, 4, 0, FAKE, None), 1),  # device count not 8-byte aligned
    ((FAKE, 2, 1, FAKE, FAKE, -1, 0, FAKE, None), 1),  # negative bound
    ((FAKE, 0, 1, FAKE, FAKE, 4, 3, FAKE, None), 2),   # MEAN of u32
    ((FAKE, 2, 1, None, FAKE, 4, 0, FAKE, None), 1),   # null offsets
    ((None, 2, 1, None, FAKE, 0, 0, None, None), 0),   # bound 0 enqueues nothing
])
def test_reduce_device_count_argument_checks(args, expect):
    lib = _lib()
    assert lib.segred_reduce_device_count(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    # (keys, n, values, lengths, offsets, count) -> status
    ((FAKE, -1, FAKE, FAKE, FAKE, FAKE), 1),
    ((FAKE, 2 ** 32, FAKE, FAKE, FAKE, FAKE), 1),      # lengths are uint32
    ((None, 5, FAKE, FAKE, FAKE, FAKE), 1),
    ((FAKE, 5, None, FAKE, FAKE, FAKE), 1),
    ((FAKE, 5, FAKE, None, FAKE, FAKE), 1),
    ((FAKE, 5, FAKE, FAKE, None, FAKE), 1),
    ((FAKE, 5, FAKE, FAKE, FAKE, None), 1),
    ((FAKE + 2, 5, FAKE, FAKE, FAKE, FAKE), 1),
    ((FAKE, 5, FAKE, FAKE, FAKE + 4, FAKE), 1),
    ((FAKE, 5, FAKE, FAKE, FAKE, FAKE + 4), 1),
])
def test_rle_argument_checks(args, expect):
    lib = _lib()
    assert lib.segred_offsets_from_rle(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    # (values, dtype, feat, rows, index, dim_size, op, out, arg) -> status
    ((FAKE, 2, 1, -1, FAKE, 4, 0, FAKE, None), 1),     # rows < 0
    ((FAKE, 2, 1, 8, FAKE, -1, 0, FAKE, None), 1),     # dim_size < 0
    ((FAKE, 2, 0, 8, FAKE, 4, 0, FAKE, None), 1),      # feat < 1
    ((FAKE, 3, 1, 8, FAKE, 4, 0, FAKE, None), 1),      # dtype out of range
    ((FAKE, 2, 1, 8, FAKE, 4, 4, FAKE, None), 1),      # op out of range
    ((FAKE, 0, 1, 8, FAKE, 4, 3, FAKE, None), 2),      # MEAN of u32
    ((FAKE, 2, 1, 2 ** 32 - 1, FAKE, 4, 2, FAKE, None), 2),  # rows do not fit the packed word
    ((None, 2, 1, 8, FAKE, 4, 0, FAKE, None), 1),      # null values
    ((FAKE, 2, 1, 8, None, 4, 0, FAKE, None), 1),      # null index
    ((FAKE, 2, 1, 8, FAKE, 4, 0, None, None), 1),      # null out
    ((FAKE + 2, 2, 1, 8, FAKE, 4, 0, FAKE, None), 1),  # values not 4-byte aligned
    ((FAKE, 2, 1, 8, FAKE + 4, 4, 0, FAKE, None), 1),  # index not 8-byte aligned
    ((FAKE, 2, 1, 8, FAKE, 4, 1, FAKE, FAKE + 4), 1),  # arg not 8-byte aligned
    ((FAKE, 2, 2 ** 40, 8, FAKE, 2 ** 40, 0, FAKE, None), 1),  # dim_size * feat overflows
    ((None, 2, 1, 0, None, 0, 0, None, None), 0),      # nothing to do
    ((FAKE, 2, 3, 8, FAKE, 0, 2, None, None), 0),      # dim_size == 0 writes nothing
])
def test_scatter_argument_checks(args, expect):
    lib = _lib()
    assert lib.segred_scatter_reduce(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    # (index, rows, dim_size, offsets) -> status
    ((FAKE, -1, 4, FAKE), 1),
    ((FAKE, 4, -1, FAKE), 1),
    ((None, 4, 4, FAKE), 1),
    ((FAKE, 4, 4, None), 1),
    ((FAKE + 4, 4, 4, FAKE), 1),
    ((FAKE, 4, 4, FAKE + 4), 1),
])
def test_offsets_from_index_argument_checks(args, expect):
    lib = _lib()
    assert lib.segred_offsets_from_index(*args, None) == expect


@pytest.mark.parametrize("fn,args,expect", [
    # (keys, n, values, count) for unique; (flags, n, offsets, count) for flags
    ("segred_unique", (FAKE, -1, FAKE, FAKE), 1),
    ("segred_unique", (FAKE, 2 ** 40 + 1, FAKE, FAKE), 1),
    ("segred_unique", (None, 5, FAKE, FAKE), 1),
    ("segred_unique", (FAKE, 5, None, FAKE), 1),
    ("segred_unique", (FAKE, 5, FAKE, None), 1),
    ("segred_unique", (FAKE + 2, 5, FAKE, FAKE), 1),
    ("segred_unique", (FAKE, 5, FAKE + 2, FAKE), 1),
    ("segred_unique", (FAKE, 5, FAKE, FAKE + 4), 1),
    ("segred_offsets_from_flags", (FAKE, -1, FAKE, FAKE), 1),
    ("segred_offsets_from_flags", (FAKE, 2 ** 40 + 1, FAKE, FAKE), 1),
    ("segred_offsets_from_flags", (None, 5, FAKE, FAKE), 1),
    ("segred_offsets_from_flags", (FAKE, 5, None, FAKE), 1),
    ("segred_offsets_from_flags", (FAKE, 5, FAKE, None), 1),
    ("segred_offsets_from_flags", (FAKE + 2, 5, FAKE, FAKE), 1),
    ("segred_offsets_from_flags", (FAKE, 5, FAKE + 4, FAKE), 1),
    ("segred_offsets_from_flags", (FAKE, 5, FAKE, FAKE + 4), 1),
])
def test_unique_and_flags_argument_checks(fn, args, expect):
    lib = _lib()
    assert getattr(lib, fn)(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    # (values, dtype, feat, offsets, S, op, exclusive, out) -> status
    ((FAKE, 2, 1, FAKE, -1, 0, 0, FAKE), 1),           # S < 0
    ((FAKE, 2, 0, FAKE, 4, 0, 0, FAKE), 1),            # feat < 1
    ((FAKE, 3, 1, FAKE, 4, 0, 0, FAKE), 1),            # dtype out of range
    ((FAKE, 2, 1, FAKE, 4, 4, 0, FAKE), 1),            # op out of range
    ((FAKE, 2, 1, FAKE, 4, 3, 0, FAKE), 2),            # MEAN has no scan
    ((FAKE, 2, 2 ** 24 + 1, FAKE, 4, 0, 0, FAKE), 2),  # too many features
    ((None, 2, 1, FAKE, 4, 0, 0, FAKE), 1),
    ((FAKE, 2, 1, None, 4, 0, 1, FAKE), 1),
    ((FAKE, 2, 1, FAKE, 4, 0, 1, None), 1),
    ((FAKE + 2, 2, 1, FAKE, 4, 1, 0, FAKE), 1),
    ((FAKE, 2, 1, FAKE + 4, 4, 1, 0, FAKE), 1),
    ((FAKE, 2, 1, FAKE, 4, 2, 0, FAKE + 2), 1),
    ((None, 2, 1, None, 0, 0, 0, None), 0),            # S == 0 enqueues nothing
])
def test_scan_argument_checks(args, expect):
    lib = _lib()
    assert lib.segred_scan(*args, None) == expect


def _gs(**kw):
    args = dict(values=FAKE, dtype=2, value_count=10, stride=1, order=None, order_count=0, queries=FAKE,
                query_count=4, segments=FAKE, S=1, max_qc=4, T=32, out=FAKE, validation=FAKE, preserve=0)
    args.update(kw)
    return tuple(args.values())


@pytest.mark.parametrize("args,expect", [
    (_gs(dtype=3), 1), (_gs(dtype=1), 2),               # unknown dtype; int32 is not searched
    (_gs(value_count=-1), 1), (_gs(stride=0), 1), (_gs(query_count=-1), 1), (_gs(S=-1), 1),
    (_gs(max_qc=-1), 1), (_gs(T=0), 1), (_gs(order=FAKE, order_count=-1), 1),
    (_gs(validation=None), 1), (_gs(segments=None), 1), (_gs(values=None), 1), (_gs(queries=None), 1),
    (_gs(out=None), 1), (_gs(values=FAKE + 2), 1), (_gs(queries=FAKE + 2), 1), (_gs(segments=FAKE + 4), 1),
    (_gs(out=FAKE + 4), 1), (_gs(validation=FAKE + 2), 1), (_gs(order=FAKE + 2, order_count=3), 1),
])
def test_galloping_argument_checks(args, expect):
    lib = _lib()
    assert lib.segred_galloping_search(*args, None) == expect


def test_share_knob_range():
    lib = _lib()
    assert lib.segred_set_shares(-1) == 1
    assert lib.segred_set_shares(2 ** 22 + 1) == 1
    assert lib.segred_set_shares(37) == 0
    assert lib.segred_get_shares(2, 0, 1) == 40  # rounded up to whole workgroups of 4 waves
    assert lib.segred_set_shares(0) == 0


# The default share count of each kernel: one share per wave of a whole
# MI355X (1,024 SIMDs x the waves per SIMD the kernel is built for), the same
# on every device, so float sums repeat across devices and partition modes.
@pytest.mark.parametrize("dtype,op,feat,shares", [
    (2, 0, 1, 2048), (2, 3, 1, 2048), (0, 0, 1, 2048), (2, 1, 1, 2048), (1, 2, 1, 2048),
    (2, 0, 32, 4096), (2, 2, 32, 4096), (2, 3, 32, 4096), (2, 0, 24, 2048), (2, 0, 8, 2048), (0, 1, 3, 2048),
    (2, 0, 16, 2048), (1, 2, 4, 2048),
    (2, 0, 64, 2048), (2, 2, 64, 2048), (2, 0, 260, 2048), (2, 0, 33, 2048), (1, 1, 100, 2048),
])
def test_default_share_counts_are_constants(dtype, op, feat, shares):
    lib = _lib()
    assert lib.segred_set_shares(0) == 0
    assert lib.segred_get_shares(dtype, op, feat) == shares
    assert lib.segred_get_shares(dtype, op, 0) == -1


def test_timing_read_without_launches():
    lib = _lib()
    ms, n = ctypes.c_double(-1.0), ctypes.c_int64(-1)
    assert lib.segred_timing_read(ctypes.byref(ms), ctypes.byref(n), None, 0) == 0
    assert n.value == 0 and ms.value == 0.0
    assert lib.segred_timing_read(None, None, None, 0) == 1
    assert lib.segred_timing_read(ctypes.byref(ms), ctypes.byref(n), None, 4) == 1


@pytest.mark.parametrize("args,expect", [
    # (src, bytes, dst, write_every, wave_sums, waves) -> status
    ((FAKE, 1000, None, 0, FAKE, 4), 1),          # not whole 1 KB blocks
    ((FAKE, 0, None, 0, FAKE, 4), 1),             # empty
    ((FAKE, 1024, None, 0, FAKE, 0), 1),          # no wave
    ((FAKE, 1024, None, 0, FAKE, 2 ** 20 + 1), 1),
    ((FAKE, 1024, None, -1, FAKE, 4), 1),
    ((FAKE, 1024, FAKE, 1025, FAKE, 4), 1),
    ((FAKE, 1024, None, 2, FAKE, 4), 1),          # writes without dst
    ((None, 1024, None, 0, FAKE, 4), 1),
    ((FAKE, 1024, None, 0, None, 4), 1),
    ((FAKE + 4, 1024, None, 0, FAKE, 4), 1),      # src not 16-byte aligned
    ((FAKE, 1024, FAKE + 4, 1, FAKE, 4), 1),
    ((FAKE, 1024, None, 0, FAKE + 2, 4), 1),
    ((FAKE, 2 ** 31, None, 0, FAKE, 1), 1),       # a share of 2 GiB
])
def test_probe_argument_checks(args, expect):
    lib = _lib()
    assert lib.segred_probe_stream(*args, None) == expect


def test_binding_refuses_cpu_tensors():
    import torch
    import segmented_reduction_amd as sr
    with pytest.raises(ValueError):
        sr.reduce(torch.zeros(4), torch.zeros(2, dtype=torch.int64), "sum")
    with pytest.raises(ValueError):
        sr.reduce(torch.zeros(4), torch.zeros(2, dtype=torch.int64), "median")


def test_kernel_sources_have_no_atomics_or_foreign_backends():
    """No atomics on global memory in the segmented and RLE paths (results are
    combined in a fixed order instead) and no CUDA/Triton/dual-platform code
    in the library sources.  The scatter path (scatter.hip) is atomic by
    definition, and the lower-bound search (galloping.hip) sets validation
    bits with an atomic OR; those two files are exempt.  Elsewhere the one atomic allowed
    is the wave-scope LDS bit-OR helper `lds_or` (it sets flag bits, so
    arrival order cannot change a result)."""
    device_atomic = re.compile(r"\batomic[A-Z]\w*\s*\(|__hip_atomic|__atomic_\w+\s*\(|\bunsafeAtomic")
    allowed = "__hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT)"
    seen_allowed = 0
    atomic_files = {"scatter.hip", "galloping.hip"}
    for name in os.listdir(CSRC):
        code = re.sub(r"//[^\n]*", "", open(os.path.join(CSRC, name)).read())
        for bad in ("cuda", "triton", "__hip_platform"):
            assert bad not in code.lower(), (name, bad)
        if name in atomic_files:
            assert device_atomic.search(code), name
            continue
        if name == "wave.hpp":
            seen_allowed = code.count(allowed)
            code = code.replace(allowed, "")
        assert not device_atomic.search(code), name
        for m in re.finditer(r"\blds_or\(&(\w+)\[", code):
            assert m.group(1) == "sm", (name, m.group(0))  # only the per-wave LDS mask array
    assert seen_allowed == 1


def test_product_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "segmented_reduction_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), os.path.join(dirpath, f)
