"""segred_reduce_device_count: the segment count read on the device (GPU only).

The count selects a prefix of the segments; results must equal the oracle on
that prefix (same bars as the other parity tests), rows of the outputs past
the count must stay untouched, and the composition RLE -> reduce must run
without reading the run count back.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC0DEAD


def _run(vals_np, off_np, count, op, capacity=None):
    import segmented_reduction_amd as sr
    v = gu.to_gpu(vals_np)
    o = gu.to_gpu(off_np)
    cap = off_np.size - 1 if capacity is None else capacity
    feat_shape = vals_np.shape[1:]
    odt = torch.float32 if op == "mean" else v.dtype
    out = torch.full((cap,) + feat_shape, SENTINEL, dtype=torch.int32, device="cuda").view(odt)
    arg = torch.full((cap,) + feat_shape, -7, dtype=torch.int64, device="cuda")
    cnt = torch.tensor([count], dtype=torch.int64, device="cuda")
    sr.reduce(v, o[: cap + 1], op, out=out, arg=arg if op in ("min", "max") else None, num_segments=cnt)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(cap, -1), arg.cpu().numpy().reshape(cap, -1)


@pytest.mark.parametrize("feat", [1, 5, 64])
@pytest.mark.parametrize("kind", ["u32", "i32", "f32"])
def test_prefix_of_segments(kind, feat):
    off, vals = W.ragged(seed=300 + feat, segments=3000, mean_len=9, feat=feat, dtype=kind, base=4,
                         long_segment=4000, tail_rows=2)
    for count in (0, 1, 1234, 3000, 5000, -3):
        s = min(max(count, 0), 3000)
        for op in ["sum", "min", "max"] + (["mean"] if kind == "f32" else []):
            gu.say(f"device count kind={kind} F={feat} count={count} op={op}")
            out, arg = _run(vals, off, count, op)
            tail = out[s:].view(np.int32)
            assert (tail == SENTINEL).all(), "rows past the count were written"
            if op in ("min", "max"):
                assert (arg[s:] == -7).all()
            if s:
                sub_off = off[: s + 1]
                gu.assert_parity(vals, sub_off, op, out[:s], arg[:s] if op in ("min", "max") else None,
                                 what=f"device count {count}")


def test_rle_to_reduce_without_readback():
    import segmented_reduction_amd as sr
    cfg = W.rle_keys(n=2_000_000)
    keys = gu.to_gpu(cfg["keys"])
    pay = gu.to_gpu(cfg["u32"][: keys.numel()])
    payi = gu.to_gpu(cfg["i32"][: keys.numel()])
    gu.say("rle -> reduce on the device count")
    values, lengths, offsets, count = sr.offsets_from_rle(keys)
    s_out, _ = sr.reduce(pay, offsets, "sum", num_segments=count)
    m_out, m_arg = sr.reduce(payi, offsets, "min", num_segments=count)
    torch.cuda.synchronize()
    c = int(count.item())
    _, _, ref_off, ref_c = oracle.rle(cfg["keys"])
    assert c == ref_c
    gu.assert_parity(cfg["u32"], ref_off, "sum", s_out.cpu().numpy()[:c].reshape(c, 1), None, what="rle sum")
    gu.assert_parity(cfg["i32"], ref_off, "min", m_out.cpu().numpy()[:c].reshape(c, 1),
                     m_arg.cpu().numpy()[:c].reshape(c, 1), what="rle min")
