"""The streaming-read ceiling probe reads every 32-bit word of its buffer
exactly once: the per-workgroup wrap-around sums add up to the buffer's own
sum, for sizes that are not whole 32 KB segments and for workgroup counts from
one to more than the segments."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_attention_decode_02_amd as pa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, (8 << 20) + 16 * 37, 64 << 20])
@pytest.mark.parametrize("workgroups", [1, 7, 2048])
def test_every_word_read_once(nbytes, workgroups):
    print("read_probe: bytes=%d workgroups=%d" % (nbytes, workgroups), flush=True)
    rng = np.random.default_rng(nbytes + workgroups)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = torch.full((workgroups,), -1, dtype=torch.int32, device="cuda:0")
    pa.read_probe(buf, sink)
    got = int(sink.cpu().numpy().view(np.uint32).astype(np.uint64).sum() % (1 << 32))
    want = int(host.astype(np.uint64).sum() % (1 << 32))
    assert got == want
    if nbytes == 0:
        assert torch.count_nonzero(sink).item() == 0
