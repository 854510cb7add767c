"""GPU checks of the library's measurement aid (smoe_stream_read)."""
import numpy as np
import pytest
import torch

import fp16_verify_expert_amd as fve
from gpu_util import host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16,blocks", [(1, 1), (1000, 3), (257 * 256 + 5, 7), (1 << 16, 2048)])
def test_stream_read_checksum(n16, blocks):
    """Workgroup b reads the 16-byte chunks i with (i // 256) % blocks == b
    (grid-stride over 256 threads); its sink word is the XOR of their 32-bit
    words."""
    say(f"stream_read n16={n16} blocks={blocks}")
    rng = np.random.default_rng(n16)
    words = rng.integers(0, 2 ** 32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
    fve.smoe_stream_read(src, sink, blocks)
    torch.cuda.synchronize()
    per_chunk = np.bitwise_xor.reduce(words, axis=1)
    owner = (np.arange(n16) // 256) % blocks
    want = np.zeros(blocks, np.uint32)
    for b in range(blocks):
        sel = per_chunk[owner == b]
        want[b] = np.bitwise_xor.reduce(sel) if sel.size else 0
    assert np.array_equal(host(sink).view(np.uint32), want)
