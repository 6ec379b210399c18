"""The streaming-read measurement kernel reads every 16-byte chunk of its range exactly once.

Each wave writes the XOR of everything its lanes loaded, so the XOR of all output words equals
the XOR of all 32-bit words of the range for every launch shape (a chunk read twice, or not at
all, changes the result for random data).
"""
import numpy as np
import pytest
import torch

import weight_only_int4_w4a16_amd as w

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks,unroll", [
    (16, 1, 1), (4096, 1, 8), (4096 + 48, 3, 4), (1 << 20, 256, 2), ((1 << 20) + 16, 512, 8),
    (37 * 4096 + 224, 7, 1),
])
def test_stream_read_touches_every_chunk_once(nbytes, blocks, unroll):
    rng = np.random.default_rng(nbytes + blocks)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4 + 8, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.full((blocks * 4,), -1, dtype=torch.int32, device="cuda")
    print(f"stream_read nbytes={nbytes} blocks={blocks} unroll={unroll}", flush=True)
    w.stream_read(buf, nbytes, out, blocks, unroll)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host[: nbytes // 4])
    assert got == want
