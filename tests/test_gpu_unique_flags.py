"""Parity of the HIP distinct-adjacent-values (segred_unique) and
offsets-from-start-flags (segred_offsets_from_flags) calls with the CPU
oracle, bit for bit (GPU only)."""
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


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _unique(keys):
    import segmented_reduction_amd as sr
    gu.say(f"unique n={keys.size}")
    v, c = sr.unique(gu.to_gpu(keys))
    c = int(c.item())
    return v[:c].cpu().numpy(), c


def _flags(flags):
    import segmented_reduction_amd as sr
    gu.say(f"offsets_from_flags n={flags.size}")
    off, c = sr.offsets_from_flags(gu.to_gpu(flags))
    c = int(c.item())
    return off[: c + 1].cpu().numpy(), c


def _check_unique(keys):
    v, c = _unique(keys)
    ov, oc = oracle.unique(keys)
    assert c == oc and np.array_equal(v, ov)


def _check_flags(flags):
    off, c = _flags(flags)
    ooff, oc = oracle.offsets_from_flags(flags)
    assert c == oc and np.array_equal(off, ooff)


def test_unique_printed_examples():
    """luma.gl GPURunLengthEncode and GPUUnique: the RLE examples' values."""
    for case in _golden("run_length_encode_examples.json")["cases"]:
        v, c = _unique(np.array(case["input"], dtype=np.uint32))
        assert v.tolist() == case["values"] and c == len(case["values"])


def test_flags_printed_layouts():
    for case in _golden("segment_start_flags.json")["cases"]:
        off, c = _flags(np.array(case["flags"], dtype=np.uint32))
        assert off.tolist() == case["offsets"] and c == case["count"]


@pytest.mark.parametrize("n", [0, 1, 2, 63, 64, 65, 4095, 4096, 4097, 8192, 12289, 100_000, 1_000_003])
def test_tile_edges(n):
    rng = np.random.default_rng(n + 5)
    keys = np.repeat(rng.integers(0, 6, n), rng.integers(1, 9, n))[:n].astype(np.uint32)
    _check_unique(keys)
    for density in (0.0, 0.001, 0.2, 1.0):
        flags = (rng.random(n) < density).astype(np.uint32)
        flags *= rng.integers(1, 2 ** 32, n, dtype=np.uint64).astype(np.uint32) | np.uint32(1)  # any nonzero word
        _check_flags(flags)


def test_extremes():
    _check_unique(np.arange(50_000, dtype=np.uint32))
    _check_unique(np.full(50_000, 7, dtype=np.uint32))
    _check_unique(np.tile(np.array([0xFFFFFFFF, 0], dtype=np.uint32), 30_000))
    f = np.zeros(300_000, dtype=np.uint32)
    f[[0, 299_999]] = 1
    _check_flags(f)
    f = np.zeros(300_000, dtype=np.uint32)
    f[150_000] = 0x80000000  # one start deep inside; rows before it belong to no segment
    _check_flags(f)


def test_untouched_past_count():
    import segmented_reduction_amd as sr
    st = torch.cuda.current_stream().cuda_stream
    keys = gu.to_gpu(np.array([5, 5, 6], dtype=np.uint32))
    vals = torch.full((3,), 77, dtype=torch.int32, device="cuda").view(torch.uint32)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    assert sr.library().segred_unique(keys.data_ptr(), 3, vals.data_ptr(), cnt.data_ptr(), st) == 0
    torch.cuda.synchronize()
    assert cnt.item() == 2 and vals.view(torch.int32).tolist() == [5, 6, 77]
    flags = gu.to_gpu(np.array([0, 3, 0, 0], dtype=np.uint32))
    offs = torch.full((5,), 99, dtype=torch.int64, device="cuda")
    assert sr.library().segred_offsets_from_flags(flags.data_ptr(), 4, offs.data_ptr(), cnt.data_ptr(), st) == 0
    torch.cuda.synchronize()
    assert cnt.item() == 1 and offs.tolist() == [1, 4, 99, 99, 99]


def test_full_size_and_composition():
    """16M Zipf keys (the sort -> RLE workload): unique equals the oracle and
    the RLE's values; the run-start flags give the RLE offsets; the flags'
    offsets then drive a segmented reduction over the device-side count."""
    import segmented_reduction_amd as sr
    cfg = W.rle_keys()
    keys = cfg["keys"]
    gk = gu.to_gpu(keys)
    gu.say("unique 16M keys")
    v, c = sr.unique(gk)
    c = int(c.item())
    ov, oc = oracle.unique(keys)
    assert c == oc and np.array_equal(v[:c].cpu().numpy(), ov)
    heads = np.ones(keys.size, dtype=np.uint32)
    heads[1:] = keys[1:] != keys[:-1]
    gu.say("offsets_from_flags 16M run-start flags")
    off, cnt = sr.offsets_from_flags(gu.to_gpu(heads))
    _, _, roff, rc = oracle.rle(keys)
    assert int(cnt.item()) == rc and np.array_equal(off[: rc + 1].cpu().numpy(), roff)
    gu.say("reduce over flag offsets with the device count")
    out = torch.empty(keys.size, dtype=torch.uint32, device="cuda")
    sr.reduce(gu.to_gpu(cfg["u32"]), off, "sum", out=out, num_segments=cnt)
    torch.cuda.synchronize()
    want = oracle.reduce(cfg["u32"], roff, "sum")
    assert np.array_equal(out[:rc].cpu().numpy(), want.out[:, 0])
