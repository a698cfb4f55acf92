"""The stream reference (leapquant_stream_reference, a measurement aid that
bench.py times beside the decode step): every byte of every block is read,
checked through the per-lane checksum against the same sum on the host, and
every written row holds the lane's checksum.  Block sizes cover one partial
16 KiB batch, whole batches and a partial last batch."""
import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("rb,wb,waves,idle", [(1024, 512, 3, 0), (5 * 1024, 0, 7, 2), (16384, 1536, 5, 0),
                                              (30 * 1024, 2048, 9, 4), (48 * 1024, 512, 2, 0)])
def test_checksums_and_rows(rb, wb, waves, idle):
    rng = np.random.default_rng(rb + wb + waves)
    host = rng.integers(0, 256, waves * rb, dtype=np.uint8)
    src = torch.as_tensor(host, device=DEV)
    dst = torch.zeros(waves * wb, dtype=torch.uint8, device=DEV) if wb else None
    out = torch.full((waves, 64), -1, dtype=torch.int32, device=DEV)
    lq.leapquant_stream_reference(src, rb, dst, wb, out, idle_sleeps=idle)
    torch.cuda.synchronize()
    # lane l of wave w reads the 16 bytes at l * 16 of every 1 KiB chunk of its block
    w = host.view(np.uint32).reshape(waves, rb // 1024, 64, 4)
    x = w[..., 0] ^ w[..., 1] ^ w[..., 2] ^ w[..., 3]
    expect = (x.astype(np.uint64).sum(axis=1) & 0xFFFFFFFF).astype(np.uint32)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), expect)
    if wb:
        # each 512-byte row: lane l's checksum twice (8 bytes per lane)
        rows = dst.cpu().numpy().view(np.uint32).reshape(waves, wb // 512, 64, 2)
        np.testing.assert_array_equal(rows, np.broadcast_to(expect[:, None, :, None], rows.shape))
