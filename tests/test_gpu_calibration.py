"""The calibration kernels read exactly the bytes they claim to: each one's
per-workgroup xor of what it read against the same xor formed on the host
from the buffer's contents (a plain streaming read, and the direct
global -> LDS copies in the prefill FFN kernels' pattern and in memory
order)."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, down

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def smoe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_routing_bit_amd as m
    return m


def buffer(nbytes, seed):
    rng = np.random.default_rng(seed)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    return host, torch.from_numpy(host.view(np.int32)).to(dev())


def xor_reduce(a, axis):
    return np.bitwise_xor.reduce(a, axis=axis)


@pytest.mark.parametrize("blocks", [3, 64, 512])
def test_stream_read_reads_every_word_once(smoe, blocks):
    nbytes = (1 << 22) + 16 * 37                   # a ragged tail past whole grid strides
    host, buf = buffer(nbytes, 1)
    sink = torch.zeros(blocks, dtype=torch.int32, device=dev())
    smoe.stream_read(buf, sink)
    w = host.reshape(-1, 4)                        # 16-byte words
    blk = (np.arange(len(w)) % (blocks * 256)) // 256
    expect = np.zeros(blocks, np.uint32)
    wx = xor_reduce(w, 1)
    for b in range(blocks):
        expect[b] = xor_reduce(wx[blk == b], 0) if np.any(blk == b) else 0
    assert np.array_equal(down(sink).view(np.uint32), expect)


@pytest.mark.parametrize("row_bytes", [2048, 768])
@pytest.mark.parametrize("mode", [0, 1])
def test_dma_read_reads_its_pattern(smoe, row_bytes, mode):
    """Each wave xors, for every stage, the first word of the 16-byte piece
    each lane copied with the stage's first copy (tile 0, or the first KB)."""
    units = 37                                     # not a multiple of four: a ragged last block
    nbytes = units * 64 * row_bytes + 4096         # and bytes past the last whole unit
    host, buf = buffer(nbytes, 2 + mode)
    blocks = (units + 3) // 4
    sink = torch.full((blocks + 5,), -1, dtype=torch.int32, device=dev())
    smoe.dma_read(buf, sink, row_bytes, mode)
    nst = 64 * row_bytes // 4096
    lane = np.arange(64)
    k = np.arange(nst)[:, None]
    if mode == 0:
        off = (lane % 16) * row_bytes + 64 * k + 16 * (lane // 16)
    else:
        off = k * 4096 + 16 * lane
    expect = np.zeros(blocks, np.uint32)
    for u in range(units):
        words = host[(u * 64 * row_bytes + off) // 4]
        expect[u // 4] ^= xor_reduce(words.ravel(), 0)
    got = down(sink).view(np.uint32)
    assert np.array_equal(got[:blocks], expect)
    assert np.all(got[blocks:] == 0xFFFFFFFF)      # nothing past the grid written
