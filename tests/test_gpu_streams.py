"""Stream ordering and the per-stream scratch cache (GPU only).

Calls on one stream reuse one cached scratch buffer, which grows when a call
needs more; calls on different streams use different buffers.  Each case
checks every output against the oracle (same bars as the other parity
tests).
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(seed, segments, feat, mean_len=40):
    off, vals = W.ragged(seed, segments, mean_len, feat, "f32", empty_frac=0.1)
    return {"offsets": off, "values": vals}


def test_scratch_grows_and_shrinks_on_one_stream():
    import segmented_reduction_amd as sr
    cases = [_case(1, 50, 1), _case(2, 3000, 300), _case(3, 20, 2), _case(4, 5000, 64)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        res = []
        for c in cases:
            v, o = gu.to_gpu(c["values"]), gu.to_gpu(c["offsets"])
            res.append((c, v, o, sr.reduce(v, o, "sum"), sr.reduce(v, o, "max")))
    s.synchronize()
    for c, _, _, (so, _), (mo, ma) in res:
        n = c["offsets"].size - 1
        gu.say(f"stream reuse S={n} F={c['values'].shape[1:]}")
        gu.assert_parity(c["values"], c["offsets"], "sum", so.cpu().numpy().reshape(n, -1), None)
        gu.assert_parity(c["values"], c["offsets"], "max", mo.cpu().numpy().reshape(n, -1),
                         ma.cpu().numpy().reshape(n, -1))


def test_concurrent_streams():
    import segmented_reduction_amd as sr
    cases = [_case(10 + i, 2000 + 500 * i, [1, 64, 7, 32][i]) for i in range(4)]
    streams = [torch.cuda.Stream() for _ in cases]
    ins = [(gu.to_gpu(c["values"]), gu.to_gpu(c["offsets"])) for c in cases]
    torch.cuda.synchronize()
    outs = [None] * len(cases)
    for rep in range(3):
        for i, (st, (v, o)) in enumerate(zip(streams, ins)):
            with torch.cuda.stream(st):
                outs[i] = (sr.reduce(v, o, "sum"), sr.reduce(v, o, "min"))
    torch.cuda.synchronize()
    for c, ((so, _), (mo, ma)) in zip(cases, outs):
        n = c["offsets"].size - 1
        gu.say(f"concurrent S={n} F={c['values'].shape[1:]}")
        gu.assert_parity(c["values"], c["offsets"], "sum", so.cpu().numpy().reshape(n, -1), None)
        gu.assert_parity(c["values"], c["offsets"], "min", mo.cpu().numpy().reshape(n, -1),
                         ma.cpu().numpy().reshape(n, -1))
