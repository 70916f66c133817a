"""The streaming-read probe the benchmark reports as the measured HBM read ceiling: every
16-byte word of the buffer is read exactly once (the XOR of the per-block XORs equals the XOR
of the buffer's words), for tiny, ragged and many-block launches."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096, 3), ((1 << 20) + 48, 7), ((1 << 22) + 16, 2048)])
def test_read_probe_reads_every_word_once(nbytes, blocks):
    import quantized_kv_paged_amd as qk
    host = np.random.default_rng(nbytes).integers(0, 256, nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    parts = qk.read_probe(buf, num_blocks=blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(parts.cpu().numpy().view(np.uint32).reshape(blocks, 4), axis=0)
    want = np.bitwise_xor.reduce(host.view(np.uint32).reshape(-1, 4), axis=0)
    np.testing.assert_array_equal(got, want)
