"""The streaming-read measurement kernel reads every byte it is given: the XOR
of the words it writes equals the XOR of the buffer's 32-bit words, for grids
and sizes that leave ragged rounds."""

import numpy as np
import pytest
import torch

from moe_testlib import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words,blocks", [(4, 1), (4 * 1001, 7), (4 * 256 * 8 * 3 + 4 * 5, 3), (1 << 22, 2048),
                                          ((1 << 22) + 12, 1000)])
def test_stream_read_probe_reads_everything(words, blocks):
    import mixture_experts_routing_align_amd as moe

    log(f"stream read probe: {words} words, {blocks} blocks")
    rng = np.random.default_rng(words + blocks)
    host = rng.integers(0, 2 ** 32, size=words, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((4 * blocks,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    moe.moe_stream_read_probe(src, sink, blocks=blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
