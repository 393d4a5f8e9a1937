"""The streaming-read probe (the bench's bandwidth ceiling) reads every byte:
the XOR of its per-block checksums equals the XOR of the buffer's words,
for every launch shape the bench tries and for ragged slice counts."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks,waves,unroll", [(16, 1, 1, 1), (4096 * 16 + 48, 7, 8, 4),
                                                        (15378432, 256, 8, 4), (33103872, 512, 8, 2),
                                                        (66134016, 256, 16, 2), (1 << 20, 256, 4, 4)])
def test_probe_reads_every_word(nbytes, blocks, waves, unroll):
    import torch
    import int4_group_quantized_quant_amd as q4
    rng = np.random.default_rng(nbytes + blocks)
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
    q4.int4_probe_stream_read(buf, sink, blocks, waves, unroll)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
