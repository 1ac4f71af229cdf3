"""The read-rate calibration kernels on the GPU: every byte asked for is read exactly once, shown by the
XOR of their checksum words equalling the XOR of the 32-bit words they were given (numpy on the host);
out-of-range block ids are skipped."""
import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from tests.gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


def _xor(words):
    return int(np.bitwise_xor.reduce(np.asarray(words, dtype=np.uint32))) if len(words) else 0


@pytest.mark.parametrize("nbytes", [4, 16, 1000, (1 << 20) + 12, 33 * (1 << 20) + 4])
def test_read_stream_reads_every_word_once(nbytes):
    note(f"read stream {nbytes} bytes")
    rng = np.random.Generator(np.random.PCG64(nbytes))
    buf = rng.integers(0, 2 ** 32, (nbytes + 3) // 4 + 8, dtype=np.uint32)
    d = dev(buf)
    sink = torch.zeros(kv.READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    kv.kv_read_stream(d, sink, nbytes=nbytes)
    torch.cuda.synchronize()
    assert _xor(host(sink, np.uint32)) == _xor(buf[:nbytes // 4])


@pytest.mark.parametrize("block_bytes,n_ids", [(2048, 1), (2048, 5000), (4096, 777), (16, 300), (1040, 64)])
def test_read_blocks_reads_the_listed_blocks(block_bytes, n_ids):
    note(f"read blocks {block_bytes} x {n_ids}")
    rng = np.random.Generator(np.random.PCG64(block_bytes + n_ids))
    nb = 3000
    buf = rng.integers(0, 2 ** 32, nb * block_bytes // 4, dtype=np.uint32)
    ids = rng.integers(0, nb, n_ids).astype(np.int32)
    if n_ids > 10:
        ids[3], ids[7] = -1, nb + 5                         # skipped, never dereferenced
    sink = torch.zeros(kv.READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    kv.kv_read_blocks(dev(buf), block_bytes, dev(ids), sink)
    torch.cuda.synchronize()
    blocks = buf.reshape(nb, block_bytes // 4)
    valid = ids[(ids >= 0) & (ids < nb)]
    assert _xor(host(sink, np.uint32)) == _xor(blocks[valid].ravel())
