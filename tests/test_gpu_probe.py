"""The streaming-rate probe (segred_probe_stream) reads and writes exactly
what its contract says: every wave's total, and for each written block the
lanes' running sums up to the input block that precedes it (GPU only).

Inputs are small integers stored as float32, so every sum is exact and the
expected values follow from the contract by integer arithmetic on the host."""
import numpy as np
import pytest
import torch

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _expected(data, waves, wevery):
    """Wave totals and written blocks, from the contract: wave w reads blocks
    [nblk*w//waves, nblk*(w+1)//waves) of 64 lanes x 4 floats; after block b
    with (b + 1) % wevery == 0 it writes each lane's running sum (x4) to
    output block b // wevery."""
    blk = data.reshape(-1, 64, 4).astype(np.int64).sum(axis=2)  # [nblk, 64] per-lane block sums
    nblk = blk.shape[0]
    sums = np.zeros(waves, dtype=np.int64)
    nout = nblk // wevery if wevery else 0
    out = np.full((nout, 64), -1, dtype=np.int64)
    for w in range(waves):
        jb, je = nblk * w // waves, nblk * (w + 1) // waves
        run = np.cumsum(blk[jb:je], axis=0)
        sums[w] = int(run[-1].sum()) if je > jb else 0
        if wevery:
            for b in range(jb, je):
                if (b + 1) % wevery == 0:
                    out[b // wevery] = run[b - jb]
    return sums, out


@pytest.mark.parametrize("nblk,waves,wevery", [
    (1, 1, 0), (1, 4, 1), (37, 4, 0), (37, 5, 3), (300, 7, 16), (300, 1024, 1), (4096, 64, 16),
    (4099, 2048, 5), (1000, 4096, 1024), (1000, 4096, 7),
])
def test_probe_contract(nblk, waves, wevery):
    import segmented_reduction_amd as sr
    rng = np.random.default_rng(nblk * 7919 + waves * 31 + wevery)
    data = rng.integers(0, 4, size=nblk * 256).astype(np.float32)
    gu.say(f"probe nblk={nblk} waves={waves} write_every={wevery}")
    src = gu.to_gpu(data)
    dst = None
    if wevery:
        # one spare block past the contract's size, filled with a sentinel
        dst = torch.full(((nblk // wevery + 1) * 256,), -1.0, dtype=torch.float32, device=src.device)
    sums, _ = sr.probe_stream(src, wevery, waves, dst)
    torch.cuda.synchronize()
    want_sums, want_out = _expected(data, waves, wevery)
    assert np.array_equal(sums.cpu().numpy().astype(np.int64), want_sums)
    if wevery:
        got = dst.cpu().numpy().reshape(-1, 64, 4)
        assert (got == got[:, :, :1]).all()  # each lane writes its sum four times
        nout = nblk // wevery
        assert np.array_equal(got[:nout, :, 0].astype(np.int64), want_out)
        assert (got[nout:] == -1.0).all()  # nothing past the contract's blocks


def test_probe_rejects_bad_sizes():
    import segmented_reduction_amd as sr
    src = torch.zeros(1000, dtype=torch.float32, device="cuda")  # 4,000 bytes: not whole blocks
    with pytest.raises(sr.SegredError):
        sr.probe_stream(src, 0, 4)
    src = torch.zeros(256, dtype=torch.float32, device="cuda")
    with pytest.raises(sr.SegredError):
        sr.probe_stream(src, 0, 0)
    with pytest.raises(sr.SegredError):
        sr.probe_stream(src, 1025, 4, torch.zeros(256, dtype=torch.float32, device="cuda"))
