"""Helpers for the GPU parity tests: run the HIP path through the C ABI (via
the binding) and compare with the CPU oracle on the same seeded inputs.

Bars (stated per call site):
  - integer sums, min/max values and their rows: bit for bit;
  - float32 sums: |gpu - ref| <= 1e-5 * sum|x| + 1e-6 per (segment, feature),
    ref and sum|x| from the oracle in float64;
  - float32 means: the same bound divided by the segment length.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TORCH = {np.dtype(np.uint32): torch.uint32, np.dtype(np.int32): torch.int32,
         np.dtype(np.float32): torch.float32, np.dtype(np.int64): torch.int64}


def say(msg: str):
    """Name the case on stdout before a GPU step (survives a lost box)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def kind_of(arr: np.ndarray) -> str:
    return oracle.dtype_name(arr)


def to_gpu(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(values_np: np.ndarray, offsets_np: np.ndarray, op: str, shares: int | None = None,
            want_arg: bool = True, values_t: torch.Tensor | None = None, offsets_t: torch.Tensor | None = None):
    import segmented_reduction_amd as sr
    v = values_t if values_t is not None else to_gpu(values_np)
    o = offsets_t if offsets_t is not None else to_gpu(offsets_np)
    if shares is not None:
        sr.set_shares(shares)
    try:
        out, arg = sr.reduce(v, o, op, want_arg=want_arg)
        torch.cuda.synchronize()
    finally:
        if shares is not None:
            sr.set_shares(0)
    s = offsets_np.shape[0] - 1
    out_np = out.cpu().numpy().reshape(s, -1)
    arg_np = arg.cpu().numpy().reshape(s, -1) if arg is not None else None
    return out_np, arg_np


def assert_parity(values_np, offsets_np, op, out_np, arg_np, orc=None, what=""):
    """Compare one GPU result with the oracle; returns the oracle result."""
    kind = kind_of(values_np)
    orc = orc or oracle.reduce(values_np, offsets_np, op)
    s = offsets_np.shape[0] - 1
    assert out_np.shape == orc.out.shape, (what, out_np.shape, orc.out.shape)
    if op in ("min", "max") or kind != "f32":
        ob = out_np.view(np.uint32)
        rb = orc.out.view(np.uint32)
        if not np.array_equal(ob, rb):
            bad = np.argwhere(ob != rb)[:5]
            raise AssertionError(f"{what} {kind} {op}: values differ at {bad.tolist()}: "
                                 f"gpu {[int(ob[tuple(b)]) for b in bad]} oracle {[int(rb[tuple(b)]) for b in bad]}")
        if arg_np is not None:
            if not np.array_equal(arg_np, orc.arg):
                bad = np.argwhere(arg_np != orc.arg)[:5]
                raise AssertionError(f"{what} {kind} {op}: args differ at {bad.tolist()}: "
                                     f"gpu {[int(arg_np[tuple(b)]) for b in bad]} "
                                     f"oracle {[int(orc.arg[tuple(b)]) for b in bad]}")
        return orc
    diff = np.abs(out_np.astype(np.float64) - orc.ref)
    tol = 1e-5 * orc.mag + 1e-6
    if op == "mean":
        lens = np.diff(offsets_np).reshape(s, 1)
        tol = tol / np.maximum(lens, 1)
        # empty segments are exactly zero
        assert (out_np[lens[:, 0] == 0] == 0).all(), what
    if not (diff <= tol).all():
        bad = np.argwhere(diff > tol)[:5]
        raise AssertionError(f"{what} f32 {op}: |gpu-ref| > tol at {bad.tolist()}: "
                             f"diff {[float(diff[tuple(b)]) for b in bad]} tol {[float(tol[tuple(b)]) for b in bad]}")
    return orc


def check(values_np, offsets_np, op, shares=None, what="", want_arg=True):
    say(f"{what} op={op} dtype={kind_of(values_np)} shape={values_np.shape} S={offsets_np.shape[0] - 1} "
        f"o0={int(offsets_np[0])} shares={shares}")
    out_np, arg_np = run_gpu(values_np, offsets_np, op, shares=shares, want_arg=want_arg)
    if not want_arg:
        arg_np = None
    return assert_parity(values_np, offsets_np, op, out_np, arg_np, what=what)


def assert_arg_invariants(values_np, offsets_np, op, out_np, arg_np):
    """Arg checks that hold at any size (graph-reduce README, 'Correctness'):
    gathered back, inside the segment, and the lowest such row."""
    s = offsets_np.shape[0] - 1
    vals = values_np.reshape(values_np.shape[0], -1)
    lo = offsets_np[:-1].reshape(s, 1)
    hi = offsets_np[1:].reshape(s, 1)
    empty = (hi == lo)[:, 0]
    assert (arg_np[empty] == -1).all() and (out_np.view(np.uint32)[empty] == 0).all()
    ne = ~empty
    a = arg_np[ne]
    assert ((a >= lo[ne]) & (a < hi[ne])).all()
    feat = np.arange(vals.shape[1])[None, :]
    gathered = vals[a, np.broadcast_to(feat, a.shape)]
    assert np.array_equal(gathered.view(np.uint32), out_np[ne].view(np.uint32))
