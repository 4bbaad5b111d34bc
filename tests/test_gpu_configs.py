"""Parity at the full sizes of the benchmarked workloads (GPU only).

Same bars as the other parity tests: integer sums, min/max values and rows
bit for bit; float32 sums within 1e-5 * sum|x| + 1e-6 (means: / length).
The oracle computes every output of every workload here; the arg checks
that hold at any size (gathered back, inside the segment, lowest row) are
run on top, and each workload's first op is repeated to check that the
result repeats bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run_all(name, cfg, key, ops):
    import segmented_reduction_amd as sr
    vals = cfg[key]
    off = cfg["offsets"]
    v = gu.to_gpu(vals)
    o = gu.to_gpu(off)
    first = None
    for op in ops:
        gu.say(f"{name}: {key} {op} shape={vals.shape} S={off.size - 1}")
        out, arg = gu.run_gpu(vals, off, op, values_t=v, offsets_t=o)
        orc = gu.assert_parity(vals, off, op, out, arg, what=name)
        if arg is not None:
            gu.assert_arg_invariants(vals, off, op, out, arg)
        del orc
        if first is None:
            first = (op, out)
    op, out = first
    again, _ = sr.reduce(v, o, op)
    torch.cuda.synchronize()
    assert np.array_equal(again.cpu().numpy().reshape(out.shape).view(np.uint32), out.view(np.uint32)), \
        f"{name}: {op} did not repeat bit for bit"


def test_small_1d():
    cfg = W.small()
    _run_all("small", cfg, "f32", ["sum", "min", "max", "mean"])
    _run_all("small", cfg, "i32", ["sum", "min", "max"])


def test_message_passing_1M_x_64():
    _run_all("message", W.message(), "f32", ["sum", "max", "mean", "min"])


def test_heavy_skew_50M():
    _run_all("skew", W.skew(), "f32", ["sum", "min", "max"])


def test_power_law_32M_x_32():
    cfg = W.powerlaw()
    _run_all("powerlaw", cfg, "f32", ["sum", "mean", "max"])
