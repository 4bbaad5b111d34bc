"""segred_reduce_noalloc through the C ABI (GPU only): the allocation-free
variant of segred_reduce must give bitwise the same outputs as
segred_reduce (same kernels, same shares), on calls in a row whose second
input is smaller than the first, so leftovers of an earlier call in the fixed
scratch cannot leak into a later one.  Beyond its fixed scratch it must fail
with SEGRED_ERR_SCRATCH_LIMIT before any device work."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SCRATCH_LIMIT = 5
DT = {np.dtype(np.uint32): 0, np.dtype(np.int32): 1, np.dtype(np.float32): 2}
OPS = {"sum": 0, "min": 1, "max": 2, "mean": 3}


def _call(fn_name, vals_t, off_t, op, feat, dtype_code):
    import segmented_reduction_amd as sr
    lib = sr.library()
    s = off_t.numel() - 1
    odt = torch.float32 if op == "mean" else vals_t.dtype
    out = torch.empty((s, feat), dtype=odt, device=vals_t.device)
    out.view(torch.int32).fill_(7)  # stale contents the call must overwrite
    arg = torch.full((s, feat), -7, dtype=torch.int64, device=vals_t.device) if op in ("min", "max") else None
    stream = torch.cuda.current_stream().cuda_stream
    rc = getattr(lib, fn_name)(vals_t.data_ptr(), dtype_code, feat, off_t.data_ptr(), s, OPS[op], out.data_ptr(),
                               arg.data_ptr() if arg is not None else None, stream)
    assert rc == 0, (fn_name, rc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (arg.cpu().numpy() if arg is not None else None)


# (feat, dtype, op, first case, second (smaller) case): 1-D, team rows, wide rows
CASES = [
    (1, "f32", "sum", dict(segments=3000, mean_len=300, long_segment=200_000),
     dict(segments=500, mean_len=20)),
    (1, "i32", "min", dict(segments=4000, mean_len=100, long_segment=50_000),
     dict(segments=300, mean_len=5)),
    (32, "f32", "max", dict(segments=5000, mean_len=30, long_segment=20_000),
     dict(segments=700, mean_len=8)),
    (32, "f32", "mean", dict(segments=3000, mean_len=40, long_segment=10_000),
     dict(segments=200, mean_len=3)),
    (64, "f32", "sum", dict(segments=2000, mean_len=80, long_segment=30_000),
     dict(segments=100, mean_len=60)),
    (100, "u32", "max", dict(segments=800, mean_len=50, long_segment=5_000),
     dict(segments=60, mean_len=10)),
]


@pytest.mark.parametrize("feat,kind,op,big,small", CASES)
def test_noalloc_matches_reduce_on_two_calls(feat, kind, op, big, small):
    for i, case in enumerate((big, small)):
        off, vals = W.ragged(seed=100 + i + feat, feat=feat, dtype=kind, **case)
        gu.say(f"noalloc feat={feat} {kind} {op} call {i} segments={case['segments']}")
        v, o = gu.to_gpu(vals), gu.to_gpu(off)
        out_a, arg_a = _call("segred_reduce_noalloc", v, o, op, feat, DT[vals.dtype])
        out_b, arg_b = _call("segred_reduce", v, o, op, feat, DT[vals.dtype])
        assert np.array_equal(out_a.view(np.uint32), out_b.view(np.uint32)), (feat, op, i)
        if arg_a is not None:
            assert np.array_equal(arg_a, arg_b), (feat, op, i)
        if i == 1:
            # the smaller call also against the oracle, at the parity bar
            gu.assert_parity(vals, off, op, out_a.reshape(len(off) - 1, -1),
                             arg_a.reshape(len(off) - 1, -1) if arg_a is not None else None)


def test_noalloc_scratch_limit():
    """A row width whose partials exceed the fixed scratch is refused."""
    import segmented_reduction_amd as sr
    lib = sr.library()
    feat = 600  # 32 * 2048 + 16 * 2048 * 600 bytes > 16 MiB
    off = torch.tensor([0, 2, 3], dtype=torch.int64, device="cuda")
    vals = torch.zeros((3, feat), dtype=torch.float32, device="cuda")
    out = torch.empty((2, feat), dtype=torch.float32, device="cuda")
    gu.say("noalloc scratch limit")
    rc = lib.segred_reduce_noalloc(vals.data_ptr(), 2, feat, off.data_ptr(), 2, 0, out.data_ptr(), None,
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == SCRATCH_LIMIT
    assert "fixed scratch" in sr.status_string(rc)
    # the regular call still works for the same request
    rc = lib.segred_reduce(vals.data_ptr(), 2, feat, off.data_ptr(), 2, 0, out.data_ptr(), None,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
