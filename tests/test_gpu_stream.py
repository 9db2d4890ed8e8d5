"""GPU checks of the streaming reference kernels that bench.py times beside
the quantizers: the read kernel's checksums fold to the XOR of every 32-bit
word read, and the copy kernel copies bit for bit (ragged sizes included)."""

import numpy as np
import pytest

from tests._helpers import announce, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 32768 * 3 + 16, 1 << 26])
def test_stream_read_checksum(nbytes):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce(f"stream read {nbytes}")
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(nv._lib.STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    nv.nvfp4_stream_read(src, nbytes, sink)
    groups = min(nv._lib.STREAM_SINK_WORDS, -(-nbytes // 32768))
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32)[:groups])
    assert got == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 1 << 26])
def test_stream_copy_exact(nbytes):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce(f"stream copy {nbytes}")
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    nv.nvfp4_stream_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].sum()) == 0
