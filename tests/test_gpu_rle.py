"""Parity of the HIP run-length encoding (and the offsets it produces) with
the CPU oracle, bit for bit (GPU only)."""
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


def _gpu_rle(keys):
    import segmented_reduction_amd as sr
    gu.say(f"rle n={keys.size}")
    v, ln, off, c = sr.rle(gu.to_gpu(keys))
    return v.cpu().numpy(), ln.cpu().numpy(), off.cpu().numpy(), c


def _check(keys):
    v, ln, off, c = _gpu_rle(keys)
    ov, oln, ooff, oc = oracle.rle(keys)
    assert c == oc
    assert np.array_equal(v, ov) and np.array_equal(ln, oln) and np.array_equal(off, ooff)


def test_printed_examples():
    """luma.gl GPURunLengthEncode, 'What is run-length encoding?', 'Contract'."""
    with open(os.path.join(GOLDEN, "run_length_encode_examples.json")) as fh:
        g = json.load(fh)
    for case in g["cases"]:
        keys = np.array(case["input"], dtype=np.uint32)
        v, ln, off, c = _gpu_rle(keys)
        assert v.tolist() == case["values"]
        assert ln.tolist() == case.get("lengths", case.get("derived_lengths"))
        assert off.tolist() == case.get("offsets", case.get("derived_offsets"))


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 4095, 4096, 4097, 8191, 8192, 12289, 100_000, 1_000_003])
def test_tile_edges(n):
    rng = np.random.default_rng(n)
    keys = np.repeat(rng.integers(0, 6, n), rng.integers(1, 9, n))[:n].astype(np.uint32)
    _check(keys)


def test_all_distinct_and_all_equal():
    _check(np.arange(50_000, dtype=np.uint32))
    _check(np.full(50_000, 7, dtype=np.uint32))
    _check(np.tile(np.array([1, 2], dtype=np.uint32), 30_000))   # every key starts a run


def test_long_runs_across_many_tiles():
    keys = np.concatenate([np.full(300_000, 3), np.full(5, 4), np.full(1_000_000, 9), [1]]).astype(np.uint32)
    _check(keys)


def test_untouched_past_count():
    """Only the valid prefix is written (luma.gl 'Contract')."""
    import segmented_reduction_amd as sr
    keys = gu.to_gpu(np.array([5, 5, 6], dtype=np.uint32))
    vals = torch.full((3,), 77, dtype=torch.int32, device="cuda").view(torch.uint32)
    lens = torch.full((3,), 88, dtype=torch.int32, device="cuda").view(torch.uint32)
    offs = torch.full((4,), 99, dtype=torch.int64, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    rc = sr.library().segred_offsets_from_rle(keys.data_ptr(), 3, vals.data_ptr(), lens.data_ptr(),
                                              offs.data_ptr(), cnt.data_ptr(),
                                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert cnt.item() == 2
    assert vals.view(torch.int32).tolist() == [5, 6, 77]
    assert lens.view(torch.int32).tolist() == [2, 1, 88]
    assert offs.tolist() == [0, 2, 3, 99]


def test_empty_input():
    v, ln, off, c = _gpu_rle(np.zeros(0, dtype=np.uint32))
    assert c == 0 and off.tolist() == [0]


def test_sort_rle_reduce_config():
    """16M Zipf keys: RLE parity, then reduction over the run offsets of the
    uint32 (sum) and int32 (min) payloads, plus composition invariants."""
    import segmented_reduction_amd as sr
    cfg = W.rle_keys()
    keys = cfg["keys"]
    gk = gu.to_gpu(keys)
    gu.say("rle config: encode 16M keys")
    v, ln, off, c = sr.rle(gk)
    ov, oln, ooff, oc = oracle.rle(keys)
    assert c == oc
    assert np.array_equal(v.cpu().numpy(), ov) and np.array_equal(ln.cpu().numpy(), oln)
    assert np.array_equal(off.cpu().numpy(), ooff)
    # reduce over the runs
    for payload, op in (("u32", "sum"), ("i32", "min")):
        gu.say(f"rle config: reduce {payload} {op}")
        out, arg = sr.reduce(gu.to_gpu(cfg[payload]), off, op)
        torch.cuda.synchronize()
        gu.assert_parity(cfg[payload], ooff, op, out.cpu().numpy().reshape(-1, 1),
                         None if arg is None else arg.cpu().numpy().reshape(-1, 1), what="rle-config")
    # composition: min/max of the keys over their own runs is the run value at
    # the run's first row; the sum of ones is the run length
    for op in ("min", "max"):
        out, arg = sr.reduce(gk, off, op)
        assert torch.equal(out, v) and torch.equal(arg, off[:-1])
    ones = torch.ones(keys.size, dtype=torch.uint32, device="cuda")
    cnt, _ = sr.reduce(ones, off, "sum")
    assert torch.equal(cnt, ln)
    assert int(ln.to(torch.int64).sum()) == keys.size
    assert bool((off[1:] > off[:-1]).all())
