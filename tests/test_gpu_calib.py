"""GPU check of the measurement aid ``pa_hbm_read`` (the read-only streaming
kernel that gives the HBM read ceiling): every 16-byte piece of the buffer is
read, ragged tails included, whatever the grid size.  A single piece holding
the kernel's fold value in an otherwise zero buffer makes exactly the thread
that reads it store that value to the sink."""

import numpy as np
import pytest
import torch

import paged_kv_cache_48_amd as pa

from gpu_util import DEV

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("pieces,wg", [(1, 1), (1000, 1), (65536 + 7, 4), (1 << 20, 1024), ((1 << 20) + 333, 37)])
def test_hbm_read_reaches_every_piece(pieces, wg):
    rng = np.random.default_rng(pieces + wg)
    buf = torch.zeros(pieces * 4, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for where in sorted(set([0, pieces - 1, int(rng.integers(0, pieces))])):
        buf.zero_()
        buf[4 * where] = np.int32(np.uint32(MAGIC).view(np.int32))
        sink.zero_()
        pa.hbm_read(buf, sink, wg)
        torch.cuda.synchronize()
        assert int(sink.item()) & 0xFFFFFFFF == MAGIC, (pieces, wg, where)
    buf.zero_()
    sink.zero_()
    pa.hbm_read(buf, sink, wg)  # a fold of zeros stores nothing
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
