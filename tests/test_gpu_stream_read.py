"""The streaming-read measurement instrument (tq_stream_read), the rate the
decode's weight stream is compared with: it must read every byte of the range
once and nothing past it.  The XOR of its sink words is checked against the
XOR of the range's 32-bit words computed on the host, for one chunk, a ragged
count below one chunk per work-item of the fixed grid, exactly one and
several chunks per work-item, and the FFN-shape tile bytes; the buffer
always extends 32 random bytes past the range, which must not be read."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

GRID_CHUNKS = 2048 * 256          # 16-byte chunks one pass of the fixed grid covers
SIZES = [16, 4096 + 16, 16 * GRID_CHUNKS, 16 * (3 * GRID_CHUNKS + 3), 33_030_144]


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


@pytest.mark.parametrize("nbytes", SIZES)
def test_stream_read_checksum(tq, nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4 + 8, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).cuda()
    sink = torch.full((tq.ops.STREAM_READ_BLOCKS,), -1, dtype=torch.int32, device="cuda")
    tq.stream_read(buf, nbytes, sink=sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host[: nbytes // 4]), nbytes


def test_stream_read_empty_leaves_sink(tq):
    buf = torch.zeros(64, dtype=torch.uint8, device="cuda")
    sink = torch.full((tq.ops.STREAM_READ_BLOCKS,), 7, dtype=torch.int32, device="cuda")
    tq.stream_read(buf, 0, sink=sink)
    torch.cuda.synchronize()
    assert bool((sink == 7).all())
